"""GPU: the calls recorded into a HIP graph and replayed.

The calls enqueue kernels (and, for bf16 fwd_bwd, a fork onto a second stream
and the join back) without host synchronisation or allocation, so a serving
loop or a trainer step can capture them.  Each graph below is captured on
the caller's stream after one eager warm-up call (which also creates the
second stream), then replayed several times with eager work and
synchronisation between the replays; every replay must reproduce the eager
results bit for bit.
"""

import pytest
import torch

import bitwise_invariant_gated_amd as gdn
from gdn_synth import make_batch

from gpu_util import DEV, DevBatch, note

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _capture(run):
    """Warm up on a side stream, then capture run() into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    return graph


def _bits(x):
    return x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32)


def _busy_work():
    """Unrelated eager work between replays."""
    a = torch.randn((1024, 1024), device=DEV)
    return float((a @ a).sum())


def test_prefill_then_decode_graph_replays_bitwise():
    note("graph: prefill 3 sequences + one decode step")
    b = make_batch(701, [300, 64, 129], 4, 128, 128, dtype="bf16", h0_std=0.1)
    nxt = make_batch(702, [1, 1, 1], 4, 128, 128, dtype="bf16")
    db, d1 = DevBatch(b), DevBatch(nxt)
    shape, N, T, H = db.shape, b.num_seqs, b.total_tokens, b.num_heads
    ws_p = gdn.alloc_workspace(shape, N, T, gdn.GDN_OP_PREFILL)
    ws_d = gdn.alloc_workspace(shape, N, 0, gdn.GDN_OP_DECODE)

    def buffers():
        return (gdn.alloc_cache(shape, N), torch.empty((T, H, 128), dtype=torch.bfloat16, device=DEV),
                torch.empty((N, H, 128), dtype=torch.bfloat16, device=DEV))

    def run_into(cache, o, od):
        gdn.gdn_cpr_prefill(shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, cache, o, ws_p)
        gdn.gdn_cpr_decode_step(shape, d1.q, d1.k, d1.v, d1.g, d1.beta, cache, od, ws_d)

    ce, oe, ode = buffers()
    run_into(ce, oe, ode)
    torch.cuda.synchronize()
    cg, og, odg = buffers()
    graph = _capture(lambda: run_into(cg, og, odg))
    for rep in range(REPLAYS):
        for t in (og, odg, cg.s_run, cg.s_bnd, cg.run_log_scale, cg.tail_len):
            t.zero_()
        _busy_work()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(og), _bits(oe)), rep
        assert torch.equal(_bits(odg), _bits(ode)), rep
        for name in ("s_run", "s_bnd", "run_log_scale", "tail_len"):
            a, e = getattr(cg, name), getattr(ce, name)
            assert torch.equal(_bits(a) if a.is_floating_point() else a, _bits(e) if e.is_floating_point() else e), \
                (rep, name)


@pytest.mark.parametrize("d", [64, 128])
def test_fwd_bwd_graph_replays_bitwise(d):
    note(f"graph: fwd_bwd d={d}")
    b = make_batch(703, [700, 130, 64], 4, d, d, dtype="bf16", h0_std=0.1, with_do=True)
    db = DevBatch(b)
    shape, N, T, H = db.shape, b.num_seqs, b.total_tokens, b.num_heads
    ws = gdn.alloc_workspace(shape, N, T, gdn.GDN_OP_FWD_BWD)
    d_hT = torch.randn((N, H, d, d), generator=torch.Generator(device=DEV).manual_seed(704), device=DEV)

    def buffers():
        bf = dict(dtype=torch.bfloat16, device=DEV)
        f32 = dict(dtype=torch.float32, device=DEV)
        return dict(o=torch.empty((T, H, d), **bf), hT=torch.empty((N, H, d, d), **f32),
                    dq=torch.empty((T, H, d), **bf), dk=torch.empty((T, H, d), **bf), dv=torch.empty((T, H, d), **bf),
                    dg=torch.empty((T, H), **f32), dbeta=torch.empty((T, H), **f32),
                    dh0=torch.empty((N, H, d, d), **f32))

    def run_into(x):
        gdn.gdn_cpr_fwd_bwd(shape, db.q, db.k, db.v, db.g, db.beta, db.cu, db.h0, db.d_o, d_hT, x["o"], x["hT"],
                            x["dq"], x["dk"], x["dv"], x["dg"], x["dbeta"], x["dh0"], ws)

    e = buffers()
    run_into(e)
    torch.cuda.synchronize()
    gb = buffers()
    graph = _capture(lambda: run_into(gb))
    for rep in range(REPLAYS):
        for t in gb.values():
            t.zero_()
        _busy_work()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in e:
            assert torch.equal(_bits(gb[name]), _bits(e[name])), (rep, name)
