"""GPU: prefill continued from a cache (gdn_cpr_prefill_continue).

A sequence prefilled in segments -- the first by gdn_cpr_prefill, the rest by
gdn_cpr_prefill_continue -- must give the bits of one prefill of the whole
sequence: every output row, both states, the tail and its length.  One token
per sequence must give the bits of gdn_cpr_decode_step.  Segment lengths
cover the cases of the split: empty, inside the cached partial chunk,
exactly closing it, and running several chunks past it.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
import oracle
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, as_f64, bits, note, prefill, state_of, torch_dtype

pytestmark = pytest.mark.gpu


def segment(db: DevBatch, starts, lens):
    """Packed tensors of rows [cu[i] + starts[i], + lens[i]) of every sequence."""
    b = db.b
    rows = np.concatenate([np.arange(b.cu_seqlens[i] + s, b.cu_seqlens[i] + s + n, dtype=np.int64)
                           for i, (s, n) in enumerate(zip(starts, lens))] + [np.zeros(0, np.int64)])
    idx = torch.from_numpy(rows).to(DEV)
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(DEV)
    pick = lambda t: t.index_select(0, idx).contiguous()
    return dict(q=pick(db.q), k=pick(db.k), v=pick(db.v), g=pick(db.g), beta=pick(db.beta), cu=cu,
                rows=rows)


def run_segments(db: DevBatch, splits):
    """Prefill segment 0, continue with the others.  splits: per segment, per
    sequence, the token count.  Returns (o over all rows in packed order, cache)."""
    b = db.b
    N, H = b.num_seqs, b.num_heads
    o_all = torch.zeros((b.total_tokens, H, b.d_v), dtype=torch_dtype(b), device=DEV)
    cache = gdn.alloc_cache(db.shape, N)
    starts = np.zeros(N, np.int64)
    for si, lens in enumerate(splits):
        lens = np.asarray(lens, np.int64)
        seg = segment(db, starts, lens)
        T = int(lens.sum())
        o = torch.empty((T, H, b.d_v), dtype=torch_dtype(b), device=DEV)
        if si == 0:
            ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL)
            gdn.gdn_cpr_prefill(db.shape, seg["q"], seg["k"], seg["v"], seg["g"], seg["beta"], seg["cu"], db.h0,
                                cache, o, ws)
        else:
            ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL_CONTINUE)
            gdn.gdn_cpr_prefill_continue(db.shape, seg["q"], seg["k"], seg["v"], seg["g"], seg["beta"], seg["cu"],
                                         cache, o, ws)
        if T > 0:
            o_all[torch.from_numpy(seg["rows"]).to(DEV)] = o
        starts += lens
    return o_all, cache


def assert_cache_bitwise(c1, c2):
    assert np.array_equal(bits(c1.tail_len), bits(c2.tail_len))
    assert np.array_equal(bits(c1.s_bnd), bits(c2.s_bnd))
    assert np.array_equal(bits(c1.s_run), bits(c2.s_run))
    assert np.array_equal(bits(c1.run_log_scale), bits(c2.run_log_scale))
    tl = c1.tail_len.cpu().numpy()
    for name in ("tail_k", "tail_v", "tail_g", "tail_beta"):
        a, b = bits(getattr(c1, name)), bits(getattr(c2, name))
        for i in range(tl.shape[0]):
            for h in range(tl.shape[1]):
                n = int(tl[i, h])
                assert np.array_equal(a[i, h, :n], b[i, h, :n]), (name, i, h)


# per sequence: full length and the segment lengths (sum = full length)
CASES = [
    # seq:      0                1               2              3             4           5
    ([[10, 5, 7], [64, 1, 63], [100, 28, 200], [0, 0, 65], [63, 70, 0], [130, 0, 3]]),
    ([[1, 62, 1], [64, 64, 64], [17, 0, 0], [70, 58, 1], [0, 1, 127], [200, 56, 8]]),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_segments_equal_one_prefill(dtype, dk, dv, case):
    note(f"prefill continue {dtype} dk={dk} dv={dv} case={case}")
    segs = np.asarray(CASES[case], np.int64)  # [N, n_segments]
    lens = segs.sum(axis=1)
    b = make_batch(700 + case, list(lens), 2, dk, dv, dtype=dtype, h0_std=0.1)
    db = DevBatch(b)
    o_full, c_full = prefill(db)
    o_seg, c_seg = run_segments(db, [segs[:, j] for j in range(segs.shape[1])])
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_seg), bits(o_full))
    assert_cache_bitwise(c_seg, c_full)


def test_one_token_continuation_equals_decode():
    note("prefill continue one token == decode")
    lens = [64, 65, 127, 1, 200, 0]
    b = make_batch(710, [n + 3 for n in lens], 3, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    N = b.num_seqs
    pre = b.truncate(lens)
    dbp = DevBatch(pre)
    _, c_a = prefill(dbp)
    c_b = c_a.clone()
    ws_d = gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_DECODE)
    ws_c = gdn.alloc_workspace(db.shape, N, N, gdn.GDN_OP_PREFILL_CONTINUE)
    cu1 = torch.arange(N + 1, dtype=torch.int32, device=DEV)
    base = b.cu_seqlens[:-1].astype(np.int64) + np.asarray(lens, np.int64)
    for s in range(3):
        rows = torch.from_numpy(base + s).to(DEV)
        x = {n: getattr(db, n)[rows].contiguous() for n in ("q", "k", "v", "g", "beta")}
        o_d = torch.empty((N, 3, 128), dtype=torch.bfloat16, device=DEV)
        o_c = torch.empty_like(o_d)
        gdn.gdn_cpr_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], c_a, o_d, ws_d)
        gdn.gdn_cpr_prefill_continue(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], cu1, c_b, o_c, ws_c)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o_c), bits(o_d)), s
    assert_cache_bitwise(c_b, c_a)


def test_empty_continuation_leaves_cache():
    note("prefill continue with no tokens")
    b = make_batch(711, [70, 5, 64], 2, 64, 64, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    _, c = prefill(db)
    ref = c.clone()
    N = b.num_seqs
    ws = gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_PREFILL_CONTINUE)
    cu = torch.zeros(N + 1, dtype=torch.int32, device=DEV)
    e = torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV)
    eg = torch.empty((0, 2), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_cpr_prefill_continue(db.shape, e, e, e, eg, eg, cu, c, e, ws)
    torch.cuda.synchronize()
    for t1, t2 in zip(c.tensors(), ref.tensors()):
        assert np.array_equal(bits(t1), bits(t2))


def test_continuation_matches_oracle():
    note("prefill continue vs oracle")
    segs = np.asarray([[100, 300], [64, 1], [0, 129], [33, 31]], np.int64)
    lens = segs.sum(axis=1)
    b = make_batch(712, list(lens), 2, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    o_seg, c_seg = run_segments(db, [segs[:, 0], segs[:, 1]])
    torch.cuda.synchronize()
    o_ref, h_ref = oracle.recurrent_forward(b.q, b.k, b.v, b.g, b.beta, b.cu_seqlens, b.h0)
    assert float(np.max(np.abs(as_f64(o_seg) - o_ref))) <= 2e-2
    assert float(np.max(np.abs(as_f64(state_of(db.shape, c_seg)) - h_ref))) <= 2e-2
