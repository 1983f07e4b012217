"""GPU: gdn_cpr_wait_status reads 0 after a normal call, whatever the
workspace held before (the call's plan clears the word): a one-launch bf16
prefill (chunk products, chain and scan waiting on one another), a prefill
of more sequences than the one-launch form takes, a continuation and
fwd_bwd, each on a workspace filled with 0xff bytes beforehand."""

import pytest
import torch

import bitwise_invariant_gated_amd as gdn
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, note, torch_dtype

pytestmark = pytest.mark.gpu


def _poisoned(shape, N, T, op):
    ws = gdn.alloc_workspace(shape, N, T, op)
    ws.fill_(255)
    return ws


def _status(shape, N, T, ws):
    s = gdn.gdn_cpr_wait_status(shape, N, T, ws)
    torch.cuda.synchronize()
    return int(s.item())


@pytest.mark.parametrize("lens", [[300, 64, 129, 0, 1000], [70] * 130])
def test_prefill_wait_status_is_zero(lens):
    note(f"wait status after prefill of {len(lens)} sequences")
    b = make_batch(1701, lens, 4, 128, 128, dtype="bf16", h0_std=0.1)
    db = DevBatch(b)
    N, T = b.num_seqs, b.total_tokens
    ws = _poisoned(db.shape, N, T, gdn.GDN_OP_PREFILL)
    assert _status(db.shape, N, T, ws) != 0  # the word as poisoned
    cache = gdn.alloc_cache(db.shape, N)
    o = torch.empty((T, 4, 128), dtype=torch_dtype(b), device=DEV)
    gdn.gdn_cpr_prefill(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, cache, o, ws)
    assert _status(db.shape, N, T, ws) == 0
    # a continuation of the same sequences by 5 tokens each, on its own poisoned workspace
    c = make_batch(1702, [5] * N, 4, 128, 128, dtype="bf16")
    dc = DevBatch(c)
    wc = _poisoned(db.shape, N, c.total_tokens, gdn.GDN_OP_PREFILL_CONTINUE)
    oc = torch.empty((c.total_tokens, 4, 128), dtype=torch_dtype(c), device=DEV)
    gdn.gdn_cpr_prefill_continue(db.shape, dc.q, dc.k, dc.v, dc.g, dc.beta, dc.cu, cache, oc, wc)
    assert _status(db.shape, N, c.total_tokens, wc) == 0


def test_fwd_bwd_wait_status_is_zero():
    note("wait status after fwd_bwd")
    b = make_batch(1703, [200, 64, 1], 2, 64, 64, dtype="bf16", with_do=True)
    db = DevBatch(b)
    N, T, H, D = b.num_seqs, b.total_tokens, 2, 64
    ws = _poisoned(db.shape, N, T, gdn.GDN_OP_FWD_BWD)
    bf = dict(dtype=torch.bfloat16, device=DEV)
    o = torch.empty((T, H, D), **bf)
    dq, dk, dv = (torch.empty((T, H, D), **bf) for _ in range(3))
    dg = torch.empty((T, H), dtype=torch.float32, device=DEV)
    db_ = torch.empty((T, H), dtype=torch.float32, device=DEV)
    gdn.gdn_cpr_fwd_bwd(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, None, db.d_o, None, o, None,
                        dq, dk, dv, dg, db_, None, ws)
    assert _status(db.shape, N, T, ws) == 0


def test_waits_that_give_up_set_the_status_and_the_next_call_recovers():
    # the test hook bounds every wait at one poll: scan units that start
    # before their boundary is published (and chain items before their chunk
    # products) give up, so the call's outputs are not valid, but every
    # work-group still finishes; the status must say so, and a normal call
    # afterwards on the same workspace must read 0 and reproduce the bits
    note("forced wait give-up: status 1, then a normal call reads 0")
    from bitwise_invariant_gated_amd import _lib
    lib = _lib.load()
    b = make_batch(1704, [1024] * 5, 4, 128, 128, dtype="bf16")
    db = DevBatch(b)
    N, T = b.num_seqs, b.total_tokens
    ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL)

    def run():
        cache = gdn.alloc_cache(db.shape, N)
        o = torch.empty((T, 4, 128), dtype=torch_dtype(b), device=DEV)
        gdn.gdn_cpr_prefill(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu, None, cache, o, ws)
        return o

    ref = run()
    assert _status(db.shape, N, T, ws) == 0
    try:
        _lib.check(lib.gdn_cpr_debug_set_wait_polls(1))
        run()
        assert _status(db.shape, N, T, ws) == 1
    finally:
        _lib.check(lib.gdn_cpr_debug_set_wait_polls(0))
    again = run()
    assert _status(db.shape, N, T, ws) == 0
    assert torch.equal(again.view(torch.int16), ref.view(torch.int16))
