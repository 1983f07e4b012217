"""GPU: the comparator evaluation orders (gdn_cmp_*), which are not CPR.

Each comparator computes the same recurrence, so each matches the CPU oracle
within the bf16 tolerance.  What differs is the agreement between stages:
  - recurrent everywhere: the prefill of L + 1 tokens and the prefill of L
    tokens followed by one recurrent decode step agree bit for bit;
  - chunkwise prefill + recurrent decode ("native mixed"): the two disagree
    (the mismatch CPR removes), while each stays within tolerance of the
    oracle.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
import oracle
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, as_f64, bits, note

pytestmark = pytest.mark.gpu

LENS = [1, 63, 64, 65, 130, 0, 300]


def cmp_prefill(db, mode, h0="batch"):
    b = db.b
    N, T, H = b.num_seqs, b.total_tokens, b.num_heads
    o = torch.empty((T, H, b.d_v), dtype=torch.bfloat16, device=DEV)
    st = torch.empty((N, H, b.d_k, b.d_v), dtype=torch.float32, device=DEV)
    ws = gdn.gdn_cmp_workspace(db.shape, mode, N, T)
    gdn.gdn_cmp_prefill(db.shape, mode, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0 if h0 == "batch" else h0,
                        st, o, ws)
    return o, st


@pytest.mark.parametrize("mode", [gdn.GDN_CMP_RECURRENT, gdn.GDN_CMP_CHUNKWISE])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
def test_comparator_prefill_matches_oracle(mode, dk, dv):
    note(f"comparator prefill mode={mode} dk={dk} dv={dv}")
    b = make_batch(730, LENS, 2, dk, dv, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    o, st = cmp_prefill(db, mode)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    assert float(np.max(np.abs(as_f64(o) - o_ref))) <= 2e-2
    assert float(np.max(np.abs(as_f64(st) - h_ref))) <= 2e-2


def _last_token_split(b):
    """Batch of every sequence without its last token, and the last tokens' rows."""
    lens = [int(x) for x in b.lengths]
    keep = [n - 1 for n in lens]
    last = np.asarray(b.cu_seqlens[1:], np.int64) - 1
    return keep, last


@pytest.mark.parametrize("mode", [gdn.GDN_CMP_RECURRENT, gdn.GDN_CMP_CHUNKWISE])
def test_prefill_then_recurrent_decode(mode):
    """Recurrent everywhere: bitwise agreement.  Chunkwise + recurrent decode:
    the outputs disagree, each within tolerance of the oracle."""
    note(f"comparator prefill then decode mode={mode}")
    lens = [65, 128, 200, 64, 300]
    b = make_batch(731, lens, 16, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    keep, last = _last_token_split(b)
    o_full, st_full = cmp_prefill(db, mode)
    dbp = DevBatch(b.truncate(keep))
    _, st = cmp_prefill(dbp, mode)
    rows = torch.from_numpy(last).to(DEV)
    x = {n: getattr(db, n)[rows].contiguous() for n in ("q", "k", "v", "g", "beta")}
    o_dec = torch.empty((len(lens), 16, 128), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_cmp_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], st, o_dec)
    torch.cuda.synchronize()
    o_pre = o_full[rows]
    if mode == gdn.GDN_CMP_RECURRENT:
        assert np.array_equal(bits(o_dec), bits(o_pre))
        assert np.array_equal(bits(st), bits(st_full))
    else:
        diff = float(torch.max(torch.abs(o_dec.float() - o_pre.float())))
        print(f"native mixed: max |decode - prefill| on the last tokens = {diff:.3e}")
        assert not np.array_equal(bits(o_dec), bits(o_pre))
        o_ref, _ = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
        assert float(np.max(np.abs(as_f64(o_dec) - o_ref[last]))) <= 2e-2


def test_cpr_agrees_where_native_mixed_does_not():
    """The same split through CPR: prefill of L + 1 == prefill of L + decode, bitwise."""
    note("CPR prefill then decode (same inputs as the comparator test)")
    lens = [65, 128, 200, 64, 300]
    b = make_batch(731, lens, 16, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    keep, last = _last_token_split(b)
    N, T = b.num_seqs, b.total_tokens
    o_full = torch.empty((T, 16, 128), dtype=torch.bfloat16, device=DEV)
    c_full = gdn.alloc_cache(db.shape, N)
    gdn.gdn_cpr_prefill(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, c_full, o_full,
                        gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL))
    dbp = DevBatch(b.truncate(keep))
    c = gdn.alloc_cache(db.shape, N)
    o_p = torch.empty((dbp.b.total_tokens, 16, 128), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_cpr_prefill(db.shape, dbp.q, dbp.k, dbp.v, dbp.g, dbp.beta, dbp.cu, db.h0, c, o_p,
                        gdn.alloc_workspace(db.shape, N, dbp.b.total_tokens, gdn.GDN_OP_PREFILL))
    rows = torch.from_numpy(last).to(DEV)
    x = {n: getattr(db, n)[rows].contiguous() for n in ("q", "k", "v", "g", "beta")}
    o_dec = torch.empty((N, 16, 128), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_cpr_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], c, o_dec,
                            gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_DECODE))
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_dec), bits(o_full[rows]))


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
def test_chunkwise_decode_equals_chunkwise_prefill(dk, dv):
    """Chunkwise everywhere: each decoded token's output is the chunkwise
    prefill's output for it, bit for bit, across chunk boundaries; at a
    length that is a multiple of C the boundary state equals the prefill's
    final state.  Starts from the CPR prefill's cache (same boundary and tail)."""
    note(f"chunkwise-everywhere decode dk={dk} dv={dv}")
    pre = np.array([62, 0, 63, 64, 126, 190])
    m = 66
    full = pre + m  # 128, 66, 129, 130, 192, 256
    b = make_batch(732, list(full), 2, dk, dv, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    N = b.num_seqs
    o_full, st_full = cmp_prefill(db, gdn.GDN_CMP_CHUNKWISE)
    dbp = DevBatch(b.truncate(list(pre)))
    cache = gdn.alloc_cache(db.shape, N)
    o_p = torch.empty((max(dbp.b.total_tokens, 1), 2, dv), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_cpr_prefill(db.shape, dbp.q, dbp.k, dbp.v, dbp.g, dbp.beta, dbp.cu, db.h0, cache, o_p,
                        gdn.alloc_workspace(db.shape, N, dbp.b.total_tokens, gdn.GDN_OP_PREFILL))
    ws = gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_DECODE)
    base = b.cu_seqlens[:-1].astype(np.int64) + pre
    o_dec = torch.empty((m, N, 2, dv), dtype=torch.bfloat16, device=DEV)
    for s in range(m):
        rows = torch.from_numpy(base + s).to(DEV)
        x = {n: getattr(db, n)[rows].contiguous() for n in ("q", "k", "v", "g", "beta")}
        gdn.gdn_cmp_chunk_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], cache, o_dec[s], ws)
    torch.cuda.synchronize()
    rows_all = torch.from_numpy((base[None, :] + np.arange(m)[:, None]).reshape(-1)).to(DEV)
    ref = o_full[rows_all].view(m, N, 2, dv)
    assert np.array_equal(bits(o_dec), bits(ref))
    for i in range(N):
        if full[i] % 64 == 0:
            assert np.array_equal(bits(cache.s_bnd[i]), bits(st_full[i])), i
            assert int(cache.tail_len[i, 0]) == 0
        else:
            assert int(cache.tail_len[i, 0]) == full[i] % 64
    o_ref, _ = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    dec_rows = (base[None, :] + np.arange(m)[:, None]).reshape(-1)
    assert float(np.max(np.abs(as_f64(o_dec).reshape(m * N, 2, dv) - o_ref[dec_rows]))) <= 2e-2
