"""GPU parity: the HIP path against the CPU fp64 oracle, and the bitwise
identities CPR promises (prefill == decode, alone == packed, rerun == run).

Tolerances: fp32 inputs max|err| <= 1e-5 * max|o_ref|; bf16 inputs
max|err| <= 2e-2 (absolute), on outputs and on final states.
"""

import numpy as np
import pytest
import torch

import oracle
from gdn_synth import make_batch, workload

from gpu_util import (DevBatch, as_f64, bits, decode_rows, note, prefill, state_of, tol_for)

pytestmark = pytest.mark.gpu


def _oracle(b):
    return oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)


def _check_vs_oracle(b, o, cache, shape):
    o_ref, h_ref = _oracle(b)
    tol_o = tol_for(b, float(np.max(np.abs(o_ref))) if o_ref.size else 1.0)
    err_o = float(np.max(np.abs(as_f64(o) - o_ref))) if o_ref.size else 0.0
    s_run = as_f64(state_of(shape, cache))
    tol_s = tol_for(b, float(np.max(np.abs(h_ref))) if h_ref.size else 1.0)
    err_s = float(np.max(np.abs(s_run - h_ref))) if h_ref.size else 0.0
    assert err_o <= tol_o, (err_o, tol_o)
    assert err_s <= tol_s, (err_s, tol_s)
    return err_o, err_s


def _cache_equal(c1, c2, tail_len):
    assert np.array_equal(bits(c1.s_run), bits(c2.s_run))
    assert np.array_equal(bits(c1.run_log_scale), bits(c2.run_log_scale))
    assert np.array_equal(bits(c1.s_bnd), bits(c2.s_bnd))
    assert np.array_equal(bits(c1.tail_len), bits(c2.tail_len))
    tl = bits(c1.tail_len)
    for name in ("tail_k", "tail_v", "tail_g", "tail_beta"):
        a, b = bits(getattr(c1, name)), bits(getattr(c2, name))
        for i in range(tl.shape[0]):
            for h in range(tl.shape[1]):
                n = int(tl[i, h])
                assert np.array_equal(a[i, h, :n], b[i, h, :n]), name


def test_tiny_f32_prefill_matches_oracle_and_decode_is_bitwise():
    """B=1, T=256, H=2, d=64, C=64, fp32, zero initial state."""
    note("tiny_f32 prefill + 256 decode steps")
    b, pre, _, _ = workload("tiny_f32")
    db = DevBatch(b)
    o_p, c_p = prefill(db)
    torch.cuda.synchronize()
    _check_vs_oracle(b, o_p, c_p, db.shape)
    # decode the same 256 tokens from an empty prefill (zero-length sequence)
    b0 = b.truncate([0])
    db0 = DevBatch(b0)
    _, c_d = prefill(db0)
    o_d = decode_rows(db, np.zeros(1, np.int64), 256, c_d)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_d[:, 0]), bits(o_p))
    _cache_equal(c_p, c_d, 0)


RAGGED = [0, 1, 63, 64, 65, 130, 200]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_ragged_prefill_matches_oracle(dtype, dk, dv):
    note(f"ragged prefill {dtype} dk={dk} dv={dv}")
    b = make_batch(101, RAGGED, 2, dk, dv, dtype=dtype, h0_std=0.1)
    db = DevBatch(b)
    o, c = prefill(db)
    torch.cuda.synchronize()
    _check_vs_oracle(b, o, c, db.shape)
    tl = bits(c.tail_len)
    for i, L in enumerate(RAGGED):
        assert np.all(tl[i] == L % 64)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_continuation_is_bitwise_equal_to_prefill(dtype):
    """Prefill a prefix, decode the rest across chunk boundaries: outputs and
    the whole cache equal one prefill over the full sequences, bit for bit."""
    note(f"decode continuation {dtype}")
    full = [140, 134, 200, 75, 261]  # prefixes 70, 64, 130, 5, 191 after 70 decode steps
    steps = 70
    b = make_batch(102, full, 2, 128, 128, dtype=dtype, h0_std=0.1)
    prefix = [L - steps for L in full]
    db = DevBatch(b)
    o_full, c_full = prefill(db)
    dp = DevBatch(b.truncate(prefix))
    o_pre, c_dec = prefill(dp)
    o_dec = decode_rows(db, np.array(prefix), steps, c_dec)
    torch.cuda.synchronize()
    ob = bits(o_full)
    od = bits(o_dec)
    for i, L in enumerate(full):
        a = int(b.cu_seqlens[i])
        assert np.array_equal(od[:, i], ob[a + prefix[i]:a + L]), i
    _cache_equal(c_full, c_dec, None)


def test_alone_equals_packed_bitwise():
    note("alone vs packed")
    lens = [77, 1, 0, 128, 300, 64, 3]
    b = make_batch(103, lens, 3, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    o, c = prefill(db)
    ob = bits(o)
    for i in range(len(lens)):
        bi = b.select([i])
        oi, ci = prefill(DevBatch(bi))
        torch.cuda.synchronize()
        sl = b.seq_slice(i)
        assert np.array_equal(bits(oi), ob[sl]), i
        assert np.array_equal(bits(ci.s_run)[0], bits(c.s_run)[i]), i
        assert np.array_equal(bits(ci.run_log_scale)[0], bits(c.run_log_scale)[i]), i
        assert np.array_equal(bits(ci.s_bnd)[0], bits(c.s_bnd)[i]), i
    # reversed batch order
    order = list(range(len(lens)))[::-1]
    br = b.select(order)
    orr, cr = prefill(DevBatch(br))
    torch.cuda.synchronize()
    obr = bits(orr)
    for pos, i in enumerate(order):
        assert np.array_equal(obr[br.seq_slice(pos)], ob[b.seq_slice(i)])


def test_rerun_is_bitwise_identical():
    note("rerun determinism")
    b = make_batch(104, [500, 257, 64], 4, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    o1, c1 = prefill(db)
    o2, c2 = prefill(db)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o1), bits(o2))
    _cache_equal(c1, c2, None)


def test_cache_round_trip_through_host_continues_bitwise():
    note("cache host round trip")
    full = [150, 90]
    b = make_batch(105, full, 2, 64, 64, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    pre = [100, 40]
    _, c = prefill(DevBatch(b.truncate(pre)))
    o1 = decode_rows(db, np.array(pre), 10, c)
    host = [t.cpu() for t in c.tensors()]
    c2 = type(c)(*(t.to("cuda") for t in host))
    c3 = c.clone()
    o2 = decode_rows(db, np.array(pre) + 10, 40, c2)
    o3 = decode_rows(db, np.array(pre) + 10, 40, c3)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o2), bits(o3))
    o_full, _ = prefill(db)
    ob = bits(o_full)
    for i in range(2):
        a = int(b.cu_seqlens[i])
        assert np.array_equal(bits(o1)[:, i], ob[a + pre[i]:a + pre[i] + 10])
        assert np.array_equal(bits(o2)[:, i], ob[a + pre[i] + 10:a + pre[i] + 50])


def test_beta_zero_zero_state_outputs_exact_zero():
    note("beta=0, h0=0")
    b = make_batch(106, [130, 64], 2, 128, 128, dtype="bf16")
    b.beta[:] = 0.0
    db = DevBatch(b)
    o, c = prefill(db)
    torch.cuda.synchronize()
    assert float(torch.max(torch.abs(o.float()))) == 0.0
    assert float(torch.max(torch.abs(c.s_run))) == 0.0


def test_prefill_5x2048_matches_oracle():
    """5 x 2,048 tokens, H=16, d=128, bf16 (full oracle, about 20 s of CPU)."""
    note("prefill 5x2048 vs oracle")
    b, _, _, _ = workload("prefill_5x2048")
    db = DevBatch(b)
    o, c = prefill(db)
    torch.cuda.synchronize()
    err_o, err_s = _check_vs_oracle(b, o, c, db.shape)
    print(f"prefill_5x2048: max|o err| = {err_o:.3e}, max|state err| = {err_s:.3e}")
