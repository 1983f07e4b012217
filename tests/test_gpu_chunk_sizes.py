"""GPU: chunk lengths C = 16 and 32 (the boundary / resynchronisation period).

A chunk of C < 64 tokens is evaluated as a 64-row chunk whose rows past C are
identity steps, so every real quantity is that of a C-row chunk.  The same
promises as for C = 64 must hold: prefill within tolerance of the fp64 oracle
(which does not depend on C), decode bit-equal to prefill across the more
frequent resynchronisations, a continued prefill bit-equal to one prefill,
alone == packed, and fwd_bwd gradients within tolerance with the forward
bit-equal to prefill.
"""

import numpy as np
import pytest
import torch

import oracle
from gdn_synth import make_batch

from gpu_util import DevBatch, as_f64, bits, decode_rows, note, prefill, state_of, tol_for
from test_gpu_continue import assert_cache_bitwise, run_segments
from test_gpu_fwd_bwd import check_grads, run_fwd_bwd

pytestmark = pytest.mark.gpu

LENS = [0, 1, 15, 16, 17, 33, 64, 100, 200]


@pytest.mark.parametrize("C", [16, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_chunk_size_prefill_matches_oracle(C, dtype, dk, dv):
    note(f"prefill C={C} {dtype} dk={dk} dv={dv}")
    b = make_batch(820, LENS, 2, dk, dv, dtype=dtype, h0_std=0.1)
    db = DevBatch(b, C)
    o, c = prefill(db)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    assert float(np.max(np.abs(as_f64(o) - o_ref))) <= tol_for(b, float(np.max(np.abs(o_ref))))
    h = as_f64(state_of(db.shape, c))
    assert float(np.max(np.abs(h - h_ref))) <= tol_for(b, float(np.max(np.abs(h_ref))))
    tl = bits(c.tail_len)
    for i, L in enumerate(LENS):
        assert np.all(tl[i] == L % C), (i, L)


@pytest.mark.parametrize("C", [16, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_size_decode_equals_prefill_bitwise(C, dtype):
    note(f"decode == prefill C={C} {dtype}")
    full = np.array([140, 134, 200, 75, 261])
    steps = 70
    b = make_batch(821, list(full), 2, 128, 128, dtype=dtype, h0_std=0.1)
    pre = full - steps
    db = DevBatch(b, C)
    o_full, c_full = prefill(db)
    _, c_dec = prefill(DevBatch(b.truncate(list(pre)), C))
    o_dec = decode_rows(db, pre, steps, c_dec)
    torch.cuda.synchronize()
    ob, od = bits(o_full), bits(o_dec)
    for i, L in enumerate(full):
        a = int(b.cu_seqlens[i])
        assert np.array_equal(od[:, i], ob[a + pre[i]:a + L]), i
    assert_cache_bitwise(c_full, c_dec)


@pytest.mark.parametrize("C", [16, 32])
def test_chunk_size_continuation_and_packing_bitwise(C):
    note(f"continuation and alone == packed C={C}")
    segs = np.asarray([[40, 90], [C, 1], [0, 2 * C + 3], [C - 1, 1]], np.int64)
    lens = segs.sum(axis=1)
    b = make_batch(822, list(lens), 2, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b, C)
    o_one, c_one = prefill(db)
    o_seg, c_seg = run_segments(db, [segs[:, 0], segs[:, 1]])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_seg), bits(o_one))
    assert_cache_bitwise(c_one, c_seg)
    ob = bits(o_one)
    for i in range(len(lens)):
        oi, ci = prefill(DevBatch(b.select([i]), C))
        torch.cuda.synchronize()
        assert np.array_equal(bits(oi), ob[b.seq_slice(i)]), i
        assert np.array_equal(bits(ci.s_run)[0], bits(c_one.s_run)[i]), i
        assert np.array_equal(bits(ci.run_log_scale)[0], bits(c_one.run_log_scale)[i]), i


@pytest.mark.parametrize("C", [16, 32])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_size_fwd_bwd_matches_oracle(C, dtype):
    note(f"fwd_bwd C={C} {dtype}")
    lens = [1, C - 1, C, C + 1, 130, 0, 200]
    b = make_batch(823, lens, 2, 128, 128, dtype=dtype, h0_std=0.1, with_do=True)
    rng = np.random.default_rng(7)
    d_hT = rng.standard_normal((len(lens), 2, 128, 128)).astype(np.float32)
    db = DevBatch(b, C)
    out = run_fwd_bwd(db, d_hT)
    o_p, c_p = prefill(db)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out["o"]), bits(o_p))
    assert np.array_equal(bits(out["hT"]), bits(state_of(db.shape, c_p)))
    errs = check_grads(b, out, d_hT)
    print({n: f"{e[0]:.2e}/{e[2]:.2e}" for n, e in errs.items()})
