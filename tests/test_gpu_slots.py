"""GPU: slot-indexed caches.

With gdn_cpr_cache.slot_index set, batch entry i must read and write only
row slot_index[i] of a larger pool, and produce the bits of the same calls
on a plain cache whose row i is that sequence: through prefill, decode
(including a resynchronisation) and a prefill continuation.  Rows the batch
does not name keep their contents.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, bits, decode_rows, note, torch_dtype

pytestmark = pytest.mark.gpu


def pool_like(shape, rows, fill=3.0):
    c = gdn.alloc_cache(shape, rows)
    for t in c.tensors():
        t.fill_(fill)
    c.tail_len.fill_(7)
    return c


def prefill_into(db, cache, cu=None, q=None):
    b = db.b
    N, T = b.num_seqs, b.total_tokens
    o = torch.empty((T, b.num_heads, b.d_v), dtype=torch_dtype(b), device=DEV)
    ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL)
    gdn.gdn_cpr_prefill(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, cache, o, ws)
    return o


def row_equal(pool, row, ref, i):
    tl = int(ref.tail_len[i, 0])
    assert np.array_equal(bits(pool.tail_len[row]), bits(ref.tail_len[i]))
    assert np.array_equal(bits(pool.s_bnd[row]), bits(ref.s_bnd[i]))
    assert np.array_equal(bits(pool.s_run[row]), bits(ref.s_run[i]))
    assert np.array_equal(bits(pool.run_log_scale[row]), bits(ref.run_log_scale[i]))
    for name in ("tail_k", "tail_v", "tail_g", "tail_beta"):
        assert np.array_equal(bits(getattr(pool, name)[row])[:, :tl], bits(getattr(ref, name)[i])[:, :tl]), name


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_slot_indexed_cache_matches_plain_cache(dtype):
    note(f"slot-indexed cache {dtype}")
    full = [200, 160, 40, 130, 70]
    pre = [150, 64, 0, 100, 6]
    steps = 60  # crosses a chunk boundary for several sequences
    b = make_batch(720, full, 2, 128, 128, dtype=dtype, h0_std=0.1)
    db = DevBatch(b)
    dbp = DevBatch(b.truncate(pre))
    N = b.num_seqs
    slots = [6, 2, 7, 0, 4]
    si = torch.tensor(slots, dtype=torch.int32, device=DEV)

    ref = gdn.alloc_cache(db.shape, N)
    o_ref = prefill_into(dbp, ref)
    pool = pool_like(db.shape, 8).with_slots(si)
    o_pool = prefill_into(dbp, pool)
    torch.cuda.synchronize()
    assert np.array_equal(bits(o_pool), bits(o_ref))

    d_ref = decode_rows(db, np.array(pre), steps // 2, ref)
    d_pool = decode_rows(db, np.array(pre), steps // 2, pool)
    torch.cuda.synchronize()
    assert np.array_equal(bits(d_pool), bits(d_ref))

    # continuation of the rest
    start = np.array(pre) + steps // 2
    rest = np.array(full) - start
    rows = np.concatenate([np.arange(b.cu_seqlens[i] + start[i], b.cu_seqlens[i + 1]) for i in range(N)])
    idx = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    x = {n: getattr(db, n).index_select(0, idx).contiguous() for n in ("q", "k", "v", "g", "beta")}
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(rest)]).astype(np.int32)).to(DEV)
    T = int(rest.sum())
    ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL_CONTINUE)
    outs = []
    for c in (ref, pool):
        o = torch.empty((T, 2, 128), dtype=torch_dtype(b), device=DEV)
        gdn.gdn_cpr_prefill_continue(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], cu, c, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    assert np.array_equal(bits(outs[1]), bits(outs[0]))

    for i, r in enumerate(slots):
        row_equal(pool, r, ref, i)
    # the state written out through the row map equals the plain cache's
    st_pool = gdn.gdn_cpr_cache_state(db.shape, pool)
    st_ref = gdn.gdn_cpr_cache_state(db.shape, ref)
    torch.cuda.synchronize()
    assert st_pool.shape == st_ref.shape
    assert np.array_equal(bits(st_pool), bits(st_ref))
    for r in set(range(8)) - set(slots):  # untouched rows
        assert int(pool.tail_len[r, 0]) == 7
        assert float(pool.s_run[r].min()) == 3.0 and float(pool.s_run[r].max()) == 3.0
        assert float(pool.run_log_scale[r].min()) == 3.0 and float(pool.run_log_scale[r].max()) == 3.0
        assert float(pool.s_bnd[r].min()) == 3.0 and float(pool.s_bnd[r].max()) == 3.0
