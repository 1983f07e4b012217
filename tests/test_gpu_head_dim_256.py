"""GPU: head dims d_k = d_v = 256 (bf16 prefill, decode, continuation and fwd_bwd).

A state column's 256 keys are split over two lanes (keys 0..127 and
128..255), whose partial sums meet in one add; the scan, decode and the
continuation head all take that split, so the usual promises must hold:
prefill within tolerance of the fp64 oracle, decode bit-equal to prefill
across resynchronisations, a continued prefill bit-equal to one prefill,
alone == packed, and the written-out final state hT bit-equal to the cache's
read-out.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
import oracle
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, as_f64, bits, decode_rows, note, prefill, state_of, tol_for
from test_gpu_continue import assert_cache_bitwise, run_segments

pytestmark = pytest.mark.gpu

D = 256
LENS = [0, 1, 31, 63, 64, 65, 130, 200]


@pytest.mark.parametrize("C", [64, 32])
def test_d256_prefill_matches_oracle(C):
    note(f"d=256 prefill vs oracle C={C}")
    b = make_batch(860 + C, LENS, 2, D, D, dtype="bf16", h0_std=0.1)
    db = DevBatch(b, C)
    o, c = prefill(db)
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    err_o = float(np.max(np.abs(as_f64(o) - o_ref)))
    h = as_f64(state_of(db.shape, c))
    err_h = float(np.max(np.abs(h - h_ref)))
    print(f"d=256 C={C}: max|o err| {err_o:.3e} (max|o| {np.max(np.abs(o_ref)):.3f}), max|state err| {err_h:.3e}")
    assert err_o <= tol_for(b, float(np.max(np.abs(o_ref))))
    assert err_h <= tol_for(b, float(np.max(np.abs(h_ref))))
    tl = bits(c.tail_len)
    for i, L in enumerate(LENS):
        assert np.all(tl[i] == L % C), (i, L)


def test_d256_decode_equals_prefill_bitwise():
    note("d=256 decode == prefill")
    full = np.array([140, 134, 200, 75, 96])
    steps = 70  # every sequence crosses a chunk boundary while decoding
    b = make_batch(870, list(full), 2, D, D, dtype="bf16", h0_std=0.1)
    pre = full - steps
    db = DevBatch(b)
    o_full, c_full = prefill(db)
    _, c_dec = prefill(DevBatch(b.truncate(list(pre))))
    o_dec = decode_rows(db, pre, steps, c_dec)
    torch.cuda.synchronize()
    ob, od = bits(o_full), bits(o_dec)
    for i, L in enumerate(full):
        a = int(b.cu_seqlens[i])
        assert np.array_equal(od[:, i], ob[a + pre[i]:a + L]), i
    assert_cache_bitwise(c_full, c_dec)


def test_d256_continuation_and_packing_bitwise():
    note("d=256 continuation == one prefill; alone == packed")
    segs = np.asarray([[40, 90], [64, 1], [0, 131], [63, 1], [10, 0]], np.int64)
    lens = segs.sum(axis=1)
    b = make_batch(871, list(lens), 2, D, D, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    o_one, c_one = prefill(db)
    o_seg, c_seg = run_segments(db, [segs[:, 0], segs[:, 1]])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_seg), bits(o_one))
    assert_cache_bitwise(c_one, c_seg)
    ob = bits(o_one)
    for i in range(len(lens)):
        oi, ci = prefill(DevBatch(b.select([i])))
        torch.cuda.synchronize()
        a, e = int(b.cu_seqlens[i]), int(b.cu_seqlens[i + 1])
        assert np.array_equal(bits(oi), ob[a:e]), i
        assert np.array_equal(bits(state_of(db.shape, ci))[0], bits(state_of(db.shape, c_one))[i]), i


def test_d256_final_state_outputs_equal_cache_state():
    note("d=256 hT from prefill and decode")
    lens = [63, 126, 130, 3]  # tails 63, 62, 2, 3: the two decode steps close the first two sequences' chunks
    b = make_batch(872, [n + 2 for n in lens], 2, D, D, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    dbp = DevBatch(b.truncate(lens))
    N, H = b.num_seqs, b.num_heads
    cache = gdn.alloc_cache(dbp.shape, N)
    hT = torch.full((N, H, D, D), 7.0, dtype=torch.float32, device=DEV)
    o = torch.empty((dbp.b.total_tokens, H, D), dtype=torch.bfloat16, device=DEV)
    ws = gdn.alloc_workspace(dbp.shape, N, dbp.b.total_tokens, gdn.GDN_OP_PREFILL)
    gdn.gdn_cpr_prefill(dbp.shape, dbp.q, dbp.k, dbp.v, dbp.g, dbp.beta, dbp.cu, dbp.h0, cache, o, ws, hT=hT)
    torch.cuda.synchronize()
    assert np.array_equal(bits(hT), bits(state_of(dbp.shape, cache)))
    wsd = gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_DECODE)
    base = b.cu_seqlens[:-1].astype(np.int64) + np.asarray(lens, np.int64)
    for s in range(2):
        rows = torch.from_numpy(base + s).to(DEV)
        x = {n: getattr(db, n)[rows].contiguous() for n in ("q", "k", "v", "g", "beta")}
        od = torch.empty((N, H, D), dtype=torch.bfloat16, device=DEV)
        hd = torch.full_like(hT, 7.0)
        gdn.gdn_cpr_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], cache, od, wsd, hT=hd)
        torch.cuda.synchronize()
        assert np.array_equal(bits(hd), bits(state_of(db.shape, cache))), s


def test_d256_fwd_bwd_matches_oracle():
    """fwd_bwd at d = 256: the forward bit-equal to prefill (outputs and hT),
    the gradients within the bf16 tolerance of the oracle's analytic backward
    (d_hT given, h0 given), on ragged lengths including empty and partial
    chunks."""
    from test_gpu_fwd_bwd import check_grads, run_fwd_bwd
    note("d=256 fwd_bwd vs oracle")
    lens = [1, 63, 64, 65, 130, 0, 200]
    b = make_batch(880, lens, 2, D, D, dtype="bf16", h0_std=0.1, with_do=True)
    rng = np.random.default_rng(9)
    d_hT = rng.standard_normal((len(lens), 2, D, D)).astype(np.float32)
    db = DevBatch(b)
    out = run_fwd_bwd(db, d_hT)
    o_p, c_p = prefill(db)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out["o"]), bits(o_p))
    assert np.array_equal(bits(out["hT"]), bits(state_of(db.shape, c_p)))
    errs = check_grads(b, out, d_hT)
    print("d=256 fwd_bwd:", {n: f"{e[0]:.2e}/{e[2]:.2e}" for n, e in errs.items()})


def test_d256_fwd_bwd_rerun_identical_and_zero_upstream():
    """Reruns give identical bits; dO = 0 and no d_hT give exactly zero
    gradients."""
    from test_gpu_fwd_bwd import NAMES, run_fwd_bwd
    note("d=256 fwd_bwd rerun, zero upstream")
    b = make_batch(881, [150, 64, 17], 2, D, D, dtype="bf16", h0_std=0.1, with_do=True)
    db = DevBatch(b)
    out1 = run_fwd_bwd(db)
    out2 = run_fwd_bwd(db)
    torch.cuda.synchronize()
    for n in ("o", "hT") + NAMES:
        assert np.array_equal(bits(out1[n]), bits(out2[n])), n
    b.d_o[:] = 0.0
    out0 = run_fwd_bwd(DevBatch(b))
    torch.cuda.synchronize()
    for n in NAMES:
        assert float(torch.max(torch.abs(out0[n].float()))) == 0.0, n


def test_d256_fwd_bwd_shared_key_heads_and_short_chunks():
    """d = 256 fwd_bwd with key heads shared by pairs of value heads: dq, dk
    (group sums) against the oracle, the rest bit-equal to the run with each
    key head repeated; and with C = 32 (identity-padded rows): forward ==
    prefill bitwise, gradients against the oracle."""
    from test_gpu_fwd_bwd import check_grads, run_fwd_bwd
    from test_gpu_key_heads import repeated
    note("d=256 fwd_bwd shared key heads, C=32")
    lens = [1, 64, 130, 0, 97]
    b = make_batch(882, lens, 4, D, D, dtype="bf16", h0_std=0.1, with_do=True, num_key_heads=2)
    d_hT = np.random.default_rng(10).standard_normal((len(lens), 4, D, D)).astype(np.float32)
    out = run_fwd_bwd(DevBatch(b), d_hT)
    out_r = run_fwd_bwd(DevBatch(repeated(b)), d_hT)
    torch.cuda.synchronize()
    errs = check_grads(b, out, d_hT)
    print("d=256 grouped:", {n: f"{e[0]:.2e}/{e[2]:.2e}" for n, e in errs.items()})
    for n in ("o", "hT", "dv", "dg", "dbeta", "dh0"):
        assert np.array_equal(bits(out[n]), bits(out_r[n])), n
    lens = [1, 31, 32, 33, 100]
    b = make_batch(883, lens, 2, D, D, dtype="bf16", h0_std=0.1, with_do=True)
    db = DevBatch(b, 32)
    out = run_fwd_bwd(db)
    o_p, c_p = prefill(db)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out["o"]), bits(o_p))
    assert np.array_equal(bits(out["hT"]), bits(state_of(db.shape, c_p)))
    errs = check_grads(b, out, None)
    print("d=256 C=32:", {n: f"{e[0]:.2e}/{e[2]:.2e}" for n, e in errs.items()})
