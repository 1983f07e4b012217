"""GPU: the decode step without a workspace (gdn_cpr_decode_step_noalloc).

Its scratch is one fixed array per device inside the library, so it must give
the bits of gdn_cpr_decode_step -- outputs, final states and the whole cache --
on every call, including the call after a larger one (the array keeps the
last call's contents), batches whose filled tails are resynchronised in
several groups, and a slot-indexed cache.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, bits, note, prefill, torch_dtype

pytestmark = pytest.mark.gpu


def prefix_lengths(N, Cl, seed):
    """Per sequence a prefix whose tail is 0, Cl/2 or 1..3 short of full, so
    that over 4 decode steps most tails fill, at different steps."""
    rng = np.random.default_rng(seed)
    short = np.array([3, 2, 1, 0, Cl // 2])
    return [int(Cl * rng.integers(0, 3) + (Cl - short[i % 5]) % Cl) for i in range(N)]


def run_both(db, pre, steps, c_ws, c_na, with_hT):
    """Decode `steps` tokens per sequence through both entry points and
    compare every step's output (and final state) bit for bit."""
    b = db.b
    N, H = b.num_seqs, b.num_heads
    ws = gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_DECODE)
    base = b.cu_seqlens[:-1].astype(np.int64) + np.asarray(pre, np.int64)
    for s in range(steps):
        rows = torch.from_numpy(base + s).to(DEV)
        x = {n: getattr(db, n)[rows].contiguous() for n in ("q", "k", "v", "g", "beta")}
        o_ws = torch.empty((N, H, b.d_v), dtype=torch_dtype(b), device=DEV)
        o_na = torch.full_like(o_ws, 7.0)
        h_ws = torch.empty((N, H, b.d_k, b.d_v), dtype=torch.float32, device=DEV) if with_hT else None
        h_na = torch.full_like(h_ws, 7.0) if with_hT else None
        gdn.gdn_cpr_decode_step(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], c_ws, o_ws, ws, hT=h_ws)
        gdn.gdn_cpr_decode_step_noalloc(db.shape, x["q"], x["k"], x["v"], x["g"], x["beta"], c_na, o_na, hT=h_na)
        torch.cuda.synchronize()
        assert np.array_equal(bits(o_na), bits(o_ws)), s
        if with_hT:
            assert np.array_equal(bits(h_na), bits(h_ws)), s


def assert_cache_equal(c1, c2):
    for name, t1, t2 in zip(("s_bnd", "s_run", "tail_k", "tail_v", "tail_g", "tail_beta", "tail_len",
                             "run_log_scale"), c1.tensors(), c2.tensors()):
        assert np.array_equal(bits(t1), bits(t2)), name


# dtype, d_k, d_v, heads, chunk, (sequences of the first call, of the second)
CASES = [
    ("bf16", 128, 128, 16, 64, (80, 7)),   # 1,024 product slots: 64 sequences per resync group
    ("f32", 64, 64, 4, 64, (400, 3)),      # 1,365 slots: 341 sequences per group
    ("bf16", 128, 64, 4, 32, (20, 19)),    # one group, C = 32
    ("bf16", 256, 256, 8, 64, (70, 5)),    # 512 slots of 128 KiB: 64 sequences per group
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_decode_equals_workspace_decode(case):
    dtype, dk, dv, H, Cl, sizes = CASES[case]
    steps = 4
    for call, N in enumerate(sizes):
        note(f"noalloc decode {dtype} dk={dk} dv={dv} H={H} C={Cl} call={call} N={N}")
        pre = prefix_lengths(N, Cl, 900 + 10 * case + call)
        b = make_batch(900 + 10 * case + call, [n + steps for n in pre], H, dk, dv, dtype=dtype, h0_std=0.1)
        db = DevBatch(b, C=Cl)
        dbp = DevBatch(b.truncate(pre), C=Cl)
        if call == 0:
            # slot-indexed pool: sequence i lives in row perm[i] of N + 5 rows
            perm = np.random.default_rng(case).permutation(N + 5)[:N]
            si = torch.from_numpy(perm.astype(np.int32)).to(DEV)
            pool = gdn.alloc_cache(db.shape, N + 5).with_slots(si)
            prefill(dbp, cache=pool)
            c_ws = pool
        else:
            _, c_ws = prefill(dbp)
        c_na = c_ws.clone()
        torch.cuda.synchronize()
        run_both(db, pre, steps, c_ws, c_na, with_hT=(call == 0))
        assert_cache_equal(c_na, c_ws)


def test_noalloc_decode_rejects_too_many_pairs_before_enqueueing():
    note("noalloc decode: size limit")
    b = make_batch(950, [3, 3], 2, 64, 64, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    _, c = prefill(db)
    ref = c.clone()
    N = 32769  # 65,538 (sequence, head) pairs at H = 2
    x = torch.zeros((N, 2, 64), dtype=torch.bfloat16, device=DEV)
    gb = torch.zeros((N, 2), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(RuntimeError, match="pairs"):  # rejected on the host: nothing is read or written
        gdn.gdn_cpr_decode_step_noalloc(db.shape, x, x, x, gb, gb, c, x)
    torch.cuda.synchronize()
    assert_cache_equal(c, ref)
