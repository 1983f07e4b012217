"""GPU: the plain fp32 final state (hT) that prefill, decode, the
continuation and fwd_bwd write out themselves, checked bit for bit against
the cache's read-out (gdn_cpr_cache_state) and, through it, against the
oracle.

The final state of a sequence that ends on a chunk boundary comes from the
boundary chain, otherwise from the scan of its last chunk (or the decode
step, the continuation head, or the resynchronisation that closes a chunk);
every one of those must give the bits exp(run_log_scale) * s_run of the
cache that the same call leaves behind.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
import oracle
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, as_f64, bits, note, state_of, tol_for, torch_dtype

pytestmark = pytest.mark.gpu

LENS = [0, 1, 63, 64, 65, 128, 130, 200]


def prefill_hT(db, C):
    b = db.b
    N, T, H = b.num_seqs, b.total_tokens, b.num_heads
    cache = gdn.alloc_cache(db.shape, N)
    o = torch.empty((T, H, b.d_v), dtype=torch_dtype(b), device=DEV)
    hT = torch.full((N, H, b.d_k, b.d_v), float("nan"), dtype=torch.float32, device=DEV)
    ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL)
    gdn.gdn_cpr_prefill(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, cache, o, ws, hT=hT)
    return o, cache, hT


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv,C", [(64, 64, 64), (128, 128, 64), (128, 64, 32), (64, 128, 16)])
def test_prefill_hT_equals_cache_state_and_oracle(dtype, dk, dv, C):
    note(f"prefill hT {dtype} dk={dk} dv={dv} C={C}")
    b = make_batch(1501, LENS, 2, dk, dv, dtype=dtype, h0_std=0.1)
    db = DevBatch(b, C)
    o, cache, hT = prefill_hT(db, C)
    ref = state_of(db.shape, cache)
    torch.cuda.synchronize()
    assert np.array_equal(bits(hT), bits(ref))
    # an empty sequence's final state is its initial state, bit for bit
    assert np.array_equal(bits(hT[0]), bits(db.h0[0]))
    _, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    err = float(np.max(np.abs(as_f64(hT) - h_ref)))
    assert err <= tol_for(b, float(np.max(np.abs(h_ref)))), err


def test_prefill_hT_may_alias_h0():
    note("prefill hT aliasing h0")
    b = make_batch(1502, [64, 100, 0], 2, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    _, _, hT = prefill_hT(db, 64)
    h = db.h0.clone()
    cache = gdn.alloc_cache(db.shape, b.num_seqs)
    o = torch.empty((b.total_tokens, 2, 128), dtype=torch.bfloat16, device=DEV)
    ws = gdn.alloc_workspace(db.shape, b.num_seqs, b.total_tokens, gdn.GDN_OP_PREFILL)
    gdn.gdn_cpr_prefill(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, h, cache, o, ws, hT=h)
    torch.cuda.synchronize()
    assert np.array_equal(bits(h), bits(hT))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_hT_equals_cache_state_across_resync(dtype):
    """Decode steps with hT requested, from caches whose tails hold 0, 30, 62
    and 63 tokens, so that some steps resynchronise: hT after every step
    equals the cache's read-out, and the outputs equal decode without hT."""
    note(f"decode hT {dtype}")
    pre = [64, 30, 62, 63]
    steps = 3
    b = make_batch(1503, [n + steps for n in pre], 2, 128, 128, dtype=dtype, h0_std=0.1)
    db = DevBatch(b)
    bp = b.truncate(pre)
    dbp = DevBatch(bp)
    N = b.num_seqs
    cache_a = gdn.alloc_cache(db.shape, N)
    o_p = torch.empty((bp.total_tokens, 2, 128), dtype=torch_dtype(b), device=DEV)
    gdn.gdn_cpr_prefill(db.shape, dbp.q, dbp.k, dbp.v, dbp.g, dbp.beta, dbp.cu, dbp.h0, cache_a, o_p,
                        gdn.alloc_workspace(db.shape, N, bp.total_tokens, gdn.GDN_OP_PREFILL))
    cache_b = cache_a.clone()
    ws = gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_DECODE)
    base = b.cu_seqlens[:-1].astype(np.int64) + np.asarray(pre, np.int64)
    for s in range(steps):
        rows = torch.from_numpy(base + s).to(DEV)
        x = {n: getattr(db, n)[rows].contiguous() for n in ("q", "k", "v", "g", "beta")}
        o_a = torch.empty((N, 2, 128), dtype=torch_dtype(b), device=DEV)
        o_b = torch.empty_like(o_a)
        hT = torch.full((N, 2, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
        gdn.gdn_cpr_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], cache_a, o_a, ws, hT=hT)
        gdn.gdn_cpr_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], cache_b, o_b, ws)
        ref = state_of(db.shape, cache_a)
        torch.cuda.synchronize()
        assert np.array_equal(bits(hT), bits(ref)), s
        assert np.array_equal(bits(o_a), bits(o_b)), s
    for t1, t2 in zip(cache_a.tensors(), cache_b.tensors()):
        assert np.array_equal(bits(t1), bits(t2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_continuation_hT_equals_cache_state(dtype):
    """Continuation segments that end inside the cached partial chunk, exactly
    close it, run past it, end on a boundary, or are empty."""
    note(f"continuation hT {dtype}")
    first = [10, 64, 100, 0, 63, 130, 17]
    second = [5, 3, 28, 65, 1, 0, 111]
    b = make_batch(1504, [a + c for a, c in zip(first, second)], 2, 64, 64, dtype=dtype, h0_std=0.1)
    db = DevBatch(b)
    N = b.num_seqs
    b1 = b.truncate(first)
    db1 = DevBatch(b1)
    cache = gdn.alloc_cache(db.shape, N)
    o1 = torch.empty((b1.total_tokens, 2, 64), dtype=torch_dtype(b), device=DEV)
    gdn.gdn_cpr_prefill(db.shape, db1.q, db1.k, db1.v, db1.g, db1.beta, db1.cu, db1.h0, cache, o1,
                        gdn.alloc_workspace(db.shape, N, b1.total_tokens, gdn.GDN_OP_PREFILL))
    rows = np.concatenate([np.arange(b.cu_seqlens[i] + first[i], b.cu_seqlens[i + 1], dtype=np.int64)
                           for i in range(N)])
    idx = torch.from_numpy(rows).to(DEV)
    x = {n: getattr(db, n).index_select(0, idx).contiguous() for n in ("q", "k", "v", "g", "beta")}
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(second)]).astype(np.int32)).to(DEV)
    T2 = int(sum(second))
    o2 = torch.empty((T2, 2, 64), dtype=torch_dtype(b), device=DEV)
    hT = torch.full((N, 2, 64, 64), float("nan"), dtype=torch.float32, device=DEV)
    gdn.gdn_cpr_prefill_continue(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], cu, cache, o2,
                                 gdn.alloc_workspace(db.shape, N, T2, gdn.GDN_OP_PREFILL_CONTINUE), hT=hT)
    ref = state_of(db.shape, cache)
    torch.cuda.synchronize()
    assert np.array_equal(bits(hT), bits(ref))
    _, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    assert float(np.max(np.abs(as_f64(hT) - h_ref))) <= tol_for(b, float(np.max(np.abs(h_ref))))


def test_fwd_bwd_hT_equals_prefill_hT():
    note("fwd_bwd hT == prefill hT")
    b = make_batch(1505, [130, 64, 1, 0], 2, 128, 128, dtype="bf16", h0_std=0.1, with_do=True)
    db = DevBatch(b)
    _, _, hT_p = prefill_hT(db, 64)
    N, T, H = b.num_seqs, b.total_tokens, 2
    bf = dict(dtype=torch.bfloat16, device=DEV)
    o = torch.empty((T, H, 128), **bf)
    hT = torch.full((N, H, 128, 128), float("nan"), dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.empty((T, H, 128), **bf) for _ in range(3))
    dg, dbeta = (torch.empty((T, H), dtype=torch.float32, device=DEV) for _ in range(2))
    ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_FWD_BWD)
    gdn.gdn_cpr_fwd_bwd(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, db.d_o, None, o, hT, dq, dk,
                        dv, dg, dbeta, None, ws)
    torch.cuda.synchronize()
    assert np.array_equal(bits(hT), bits(hT_p))
