"""GPU: query and key heads shared by groups of value heads (num_key_heads).

Value head h reads key head h // G, G = H / H_k.  Per value head the library
does the arithmetic of the plain layout, so every output, final state and
cache entry equals, bit for bit, the plain layout run on q and k with each key
head repeated for its G value heads.  dq and dk are the group sums (fp32
partials summed in ascending head order, rounded once), checked against the
oracle within the usual tolerance.  Prefill == decode, segments == one
prefill, and the comparators hold as in the plain layout.
"""

import dataclasses

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
import oracle
from gdn_synth import make_batch

from gpu_util import (DEV, DevBatch, as_f64, bits, decode_rows, note, prefill, shape_of, state_of, tol_for,
                      torch_dtype)
from test_gpu_continue import assert_cache_bitwise, run_segments
from test_gpu_fwd_bwd import check_grads, run_fwd_bwd

pytestmark = pytest.mark.gpu

LENS = [1, 63, 64, 65, 130, 0, 300]


def repeated(b):
    """The same batch in the plain layout: each key head repeated per value head."""
    G = b.num_heads // b.num_key_heads
    return dataclasses.replace(b, q=np.repeat(b.q, G, axis=1), k=np.repeat(b.k, G, axis=1),
                               num_key_heads=b.num_heads)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("H,Hk", [(4, 2), (4, 1)])
def test_grouped_prefill_equals_repeated_heads_and_oracle(dtype, dk, dv, H, Hk):
    note(f"grouped prefill {dtype} dk={dk} dv={dv} H={H} Hk={Hk}")
    b = make_batch(760, LENS, H, dk, dv, dtype=dtype, h0_std=0.1, num_key_heads=Hk)
    assert b.q.shape[1] == Hk
    o, c = prefill(DevBatch(b))
    o_r, c_r = prefill(DevBatch(repeated(b)))
    torch.cuda.synchronize()
    assert np.array_equal(bits(o), bits(o_r))
    assert_cache_bitwise(c, c_r)
    o_ref, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    m = float(np.max(np.abs(o_ref)))
    assert float(np.max(np.abs(as_f64(o) - o_ref))) <= tol_for(b, m)
    h = as_f64(state_of(shape_of(b), c))
    assert float(np.max(np.abs(h - h_ref))) <= tol_for(b, float(np.max(np.abs(h_ref))))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grouped_prefill_equals_decode(dtype):
    """Prefill of L tokens + m decode steps (crossing resynchronisations) gives
    the bits of one prefill of L + m tokens."""
    note(f"grouped prefill == decode {dtype}")
    pre = np.array([0, 1, 63, 64, 100])
    m = 70
    b = make_batch(761, list(pre + m), 6, 128, 128, dtype=dtype, h0_std=0.1, num_key_heads=2)
    db = DevBatch(b)
    o_full, c_full = prefill(db)
    _, c = prefill(DevBatch(b.truncate(list(pre))), h0=db.h0)
    o_dec = decode_rows(db, pre, m, c)
    torch.cuda.synchronize()
    rows = (b.cu_seqlens[:-1].astype(np.int64)[None, :] + pre[None, :] + np.arange(m)[:, None])
    ref = o_full[torch.from_numpy(rows.reshape(-1)).to(DEV)].view(m, len(pre), 6, 128)
    assert np.array_equal(bits(o_dec), bits(ref))
    assert np.array_equal(bits(c.s_run), bits(c_full.s_run))
    assert np.array_equal(bits(c.run_log_scale), bits(c_full.run_log_scale))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_grouped_fwd_bwd(dtype):
    """Gradients against the oracle (dq, dk summed over each group); o, hT,
    dv, dg, dbeta and dh0 bit-equal to the repeated-head run."""
    note(f"grouped fwd_bwd {dtype}")
    lens = [1, 63, 64, 65, 130, 0, 200]
    b = make_batch(762, lens, 4, 64, 128, dtype=dtype, h0_std=0.1, with_do=True, num_key_heads=2)
    d_hT = np.random.default_rng(8).standard_normal((len(lens), 4, 64, 128)).astype(np.float32)
    out = run_fwd_bwd(DevBatch(b), d_hT)
    out_r = run_fwd_bwd(DevBatch(repeated(b)), d_hT)
    torch.cuda.synchronize()
    errs = check_grads(b, out, d_hT)
    print({n: f"{e[0]:.2e}/{e[2]:.2e}" for n, e in errs.items()})
    for n in ("o", "hT", "dv", "dg", "dbeta", "dh0"):
        assert np.array_equal(bits(out[n]), bits(out_r[n])), n


def test_grouped_continuation_segments_equal_one_prefill():
    note("grouped continuation")
    segs = np.asarray([[10, 5, 7], [64, 1, 63], [100, 28, 200], [0, 0, 65], [63, 70, 0]], np.int64)
    b = make_batch(763, list(segs.sum(axis=1)), 4, 128, 128, dtype="bf16", h0_std=0.1, num_key_heads=1)
    db = DevBatch(b)
    o_full, c_full = prefill(db)
    o_seg, c_seg = run_segments(db, [segs[:, j] for j in range(segs.shape[1])])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_seg), bits(o_full))
    assert_cache_bitwise(c_seg, c_full)


@pytest.mark.parametrize("mode", [gdn.GDN_CMP_RECURRENT, gdn.GDN_CMP_CHUNKWISE])
def test_grouped_comparator_prefill_equals_repeated_heads(mode):
    note(f"grouped comparator prefill mode={mode}")
    b = make_batch(764, LENS, 4, 128, 128, dtype="bf16", h0_std=0.1, num_key_heads=2)
    outs = []
    for bb in (b, repeated(b)):
        db = DevBatch(bb)
        N, T = bb.num_seqs, bb.total_tokens
        o = torch.empty((T, 4, 128), dtype=torch.bfloat16, device=DEV)
        st = torch.empty((N, 4, 128, 128), dtype=torch.float32, device=DEV)
        gdn.gdn_cmp_prefill(db.shape, mode, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, st, o,
                            gdn.gdn_cmp_workspace(db.shape, mode, N, T))
        outs.append((o, st))
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[0][0]), bits(outs[1][0]))
    assert np.array_equal(bits(outs[0][1]), bits(outs[1][1]))
