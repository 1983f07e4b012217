"""GPU: buffers past 4 GiB.

4,160 sequences x 16 heads x (128 x 128) fp32 states is 4.36 GB per state
array, and the prefill workspace (a boundary state per chunk and head) is
larger still, so every state, boundary and chunk-product offset above 2^32
bytes (and above 2^31 elements) is exercised.  Decode must still equal one
prefill bit for bit across a resynchronisation, and the last sequences (the
largest offsets) must match the fp64 oracle.  Inputs are drawn on the GPU
from a seeded generator (same distributions as the synthetic workloads); the
oracle reads back the sampled sequences.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn
import oracle

from gpu_util import DEV, as_f64, note

pytestmark = pytest.mark.gpu

N, H, D, PRE, STEPS = 4160, 16, 128, 70, 60  # decode crosses the chunk boundary at token 128


def _inputs(total, gen):
    def bf(x):
        return x.to(torch.bfloat16)
    q = torch.randn((total, H, D), generator=gen, device=DEV)
    k = torch.randn((total, H, D), generator=gen, device=DEV)
    q = bf(q / q.norm(dim=-1, keepdim=True))
    k = bf(k / k.norm(dim=-1, keepdim=True))
    v = bf(torch.randn((total, H, D), generator=gen, device=DEV))
    beta = bf(torch.sigmoid(torch.randn((total, H), generator=gen, device=DEV)))
    g = bf(-torch.nn.functional.softplus(torch.randn((total, H), generator=gen, device=DEV)) * 0.1)
    return q, k, v, g, beta


def test_states_and_workspaces_beyond_4gib():
    note(f"large: {N} sequences x {H} heads, states {N * H * D * D * 4 / 1e9:.2f} GB per array")
    L = PRE + STEPS
    gen = torch.Generator(device=DEV)
    gen.manual_seed(951)
    q, k, v, g, beta = _inputs(N * L, gen)
    shape = gdn.LayerShape(H, D, D, 64, torch.bfloat16)
    cu_full = torch.arange(0, N * L + 1, L, dtype=torch.int32, device=DEV)
    assert cu_full.numel() == N + 1
    # one prefill of all L tokens per sequence
    c_full = gdn.alloc_cache(shape, N, DEV)
    o_full = torch.empty((N * L, H, D), dtype=torch.bfloat16, device=DEV)
    ws = gdn.alloc_workspace(shape, N, N * L, gdn.GDN_OP_PREFILL, DEV)
    assert ws.numel() > 2 ** 32
    gdn.gdn_cpr_prefill(shape, q, k, v, g, beta, cu_full, None, c_full, o_full, ws)
    # prefill of the first PRE tokens, then STEPS decode steps
    rows_pre = (torch.arange(N, device=DEV)[:, None] * L + torch.arange(PRE, device=DEV)[None, :]).reshape(-1)
    cu_pre = torch.arange(0, N * PRE + 1, PRE, dtype=torch.int32, device=DEV)
    c_dec = gdn.alloc_cache(shape, N, DEV)
    o_pre = torch.empty((N * PRE, H, D), dtype=torch.bfloat16, device=DEV)
    gdn.gdn_cpr_prefill(shape, q[rows_pre].contiguous(), k[rows_pre].contiguous(), v[rows_pre].contiguous(),
                        g[rows_pre].contiguous(), beta[rows_pre].contiguous(), cu_pre, None, c_dec, o_pre, ws)
    torch.cuda.synchronize()
    assert torch.equal(o_pre.view(torch.int16), o_full[rows_pre].view(torch.int16))
    del ws, o_pre
    ws_d = gdn.alloc_workspace(shape, N, 0, gdn.GDN_OP_DECODE, DEV)
    o_d = torch.empty((N, H, D), dtype=torch.bfloat16, device=DEV)
    base = torch.arange(N, device=DEV) * L + PRE
    for s in range(STEPS):
        r = base + s
        gdn.gdn_cpr_decode_step(shape, q[r].contiguous(), k[r].contiguous(), v[r].contiguous(), g[r].contiguous(),
                                beta[r].contiguous(), c_dec, o_d, ws_d)
        assert torch.equal(o_d.view(torch.int16), o_full[r].view(torch.int16)), s
    torch.cuda.synchronize()
    for name in ("s_run", "s_bnd", "run_log_scale", "tail_len"):
        a, b = getattr(c_dec, name), getattr(c_full, name)
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b), name
    # the last sequences against the oracle
    st = gdn.gdn_cpr_cache_state(shape, c_full)
    for i in (N - 1, N - 2):
        sl = slice(i * L, (i + 1) * L)
        f = lambda t: t[sl].float().cpu().numpy()
        o_ref, h_ref = oracle.recurrent_forward(f(q), f(k), f(v), f(g), f(beta), np.array([0, L], np.int32), None)
        assert float(np.max(np.abs(as_f64(o_full[sl]) - o_ref))) <= 2e-2, i
        assert float(np.max(np.abs(as_f64(st[i:i + 1]) - h_ref))) <= 2e-2, i
