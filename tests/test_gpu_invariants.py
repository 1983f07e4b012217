"""GPU checks against what the recurrence itself fixes, with no oracle in the
loop (invariants of the update rule, applied to the HIP path directly).

- Store and retrieve: with alpha = 1 (g = 0), beta = 1 and orthonormal keys,
  writing value v_j under key k_j and then querying with q = k_j returns v_j:
  after a write, M k_j = v_j (the projection removes the old content along
  k_j and stores v_j there), and writes along orthogonal keys do not disturb
  it; a token with beta = 0 writes nothing.  The keys are the rows of a
  64 x 64 Sylvester-Hadamard matrix scaled by 1/8, orthonormal exactly in
  fp32 and bf16, so the expected outputs are exact and only the sums of
  value terms round.
- Pure decay: with beta = 0 every update is M_t = alpha_t M_{t-1}, so
  M_t = exp(g_1 + ... + g_t) h0 and o_t = exp(g_1 + ... + g_t) M_0 q_t in
  closed form (evaluated here in fp64 from the same fp32 inputs).

Tolerances: 1e-5 * max|o| for fp32 inputs and 2e-2 absolute for
bf16 inputs.
"""

import numpy as np
import pytest
import torch

import bitwise_invariant_gated_amd as gdn

from gdn_synth import round_to_bf16
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def hadamard(n):
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def run_prefill(shape, q, k, v, g, beta, lens, h0=None):
    dt = shape.dtype
    N, H = len(lens), shape.num_heads
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).to(dt).contiguous()
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(DEV)
    T = int(sum(lens))
    o = torch.empty((T, H, shape.head_dim_v), dtype=dt, device=DEV)
    hT = torch.empty((N, H, shape.head_dim_k, shape.head_dim_v), dtype=torch.float32, device=DEV)
    cache = gdn.alloc_cache(shape, N)
    h0d = None if h0 is None else torch.from_numpy(np.ascontiguousarray(h0, np.float32)).to(DEV)
    gdn.gdn_cpr_prefill(shape, t(q), t(k), t(v), t(g), t(beta), cu, h0d, cache, o,
                        gdn.alloc_workspace(shape, N, T, gdn.GDN_OP_PREFILL), hT=hT)
    return o, hT, cache


def store_retrieve_inputs(dv, H=2, seed=0, bf16=False):
    """64 writes (k_j = q_j = Hadamard row j / 8, beta = 1, g = 0), then 64
    reads (beta = 0, q = a written key, in another order).  Returns the inputs
    and the expected outputs of all 128 tokens (values rounded to bf16 first
    when bf16)."""
    rng = np.random.default_rng(seed)
    keys = hadamard(64) / 8.0
    T = 128
    q = np.empty((T, H, 64))
    k = np.empty((T, H, 64))
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    if bf16:
        v = round_to_bf16(v)
    v = v.astype(np.float64)
    g = np.zeros((T, H))
    beta = np.zeros((T, H))
    want = np.empty((T, H, dv))
    for h in range(H):
        perm_w = rng.permutation(64)
        perm_r = rng.permutation(64)
        k[:64, h] = keys[perm_w]
        q[:64, h] = keys[perm_w]
        beta[:64, h] = 1.0
        want[:64, h] = v[:64, h]
        k[64:, h] = keys[rng.permutation(64)]  # not written: beta = 0
        q[64:, h] = keys[perm_w[perm_r]]
        want[64:, h] = v[perm_r, h]
    return q, k, v, g, beta, want


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dv", [64, 128])
def test_store_and_retrieve_with_orthonormal_keys(dtype, dv):
    note(f"invariant store/retrieve {dtype} dv={dv}")
    q, k, v, g, beta, want = store_retrieve_inputs(dv, bf16=dtype == torch.bfloat16)
    shape = gdn.LayerShape(2, 64, dv, 64, dtype)
    o, hT, _ = run_prefill(shape, q, k, v, g, beta, [128])
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - want)))
    tol = 1e-5 * float(np.max(np.abs(want))) if dtype == torch.float32 else 2e-2
    assert err <= tol, (err, tol)
    # the stored state is sum_j v_j k_j^T (S = M^T: S[i][c] = sum_j k_j[i] v_j[c])
    S_want = np.einsum("thi,thc->hic", k[:64], v[:64])
    errS = float(np.max(np.abs(hT[0].cpu().numpy() - S_want)))
    assert errS <= 1e-5 * float(np.max(np.abs(S_want))), errS


def test_store_and_retrieve_through_decode():
    """The same reads through single-token decode steps from the cache after the writes."""
    note("invariant store/retrieve via decode")
    q, k, v, g, beta, want = store_retrieve_inputs(128, seed=3)
    shape = gdn.LayerShape(2, 64, 128, 64, torch.float32)
    _, _, cache = run_prefill(shape, q[:64], k[:64], v[:64], g[:64], beta[:64], [64])
    ws = gdn.alloc_workspace(shape, 1, 0, gdn.GDN_OP_DECODE)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(DEV).contiguous()
    outs = []
    for s in range(64, 128):
        o = torch.empty((1, 2, 128), dtype=torch.float32, device=DEV)
        gdn.gdn_cpr_decode_step(shape, t(q[s:s + 1]), t(k[s:s + 1]), t(v[s:s + 1]), t(g[s:s + 1]),
                                t(beta[s:s + 1]), cache, o, ws)
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.cat(outs).cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(got - want[64:])))
    assert err <= 1e-5 * float(np.max(np.abs(want))), err


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_pure_decay_closed_form(dk, dv):
    """beta = 0, nonzero h0, fp32: o_t = exp(gamma_t) M_0 q_t, final state
    exp(gamma_L) h0, with gamma_t the running sum of g."""
    note(f"invariant pure decay dk={dk} dv={dv}")
    rng = np.random.default_rng(11)
    lens = [1, 64, 65, 200]
    H = 2
    T = sum(lens)
    q = rng.standard_normal((T, H, dk)).astype(np.float32)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, dk)).astype(np.float32)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    g = (-np.logaddexp(0.0, rng.standard_normal((T, H))) * 0.1).astype(np.float32)
    beta = np.zeros((T, H), np.float32)
    h0 = (rng.standard_normal((len(lens), H, dk, dv)) * 0.1).astype(np.float32)
    shape = gdn.LayerShape(H, dk, dv, 64, torch.float32)
    o, hT, _ = run_prefill(shape, q, k, v, g, beta, lens, h0)
    torch.cuda.synchronize()
    got, gotS = o.cpu().numpy().astype(np.float64), hT.cpu().numpy().astype(np.float64)
    want = np.empty((T, H, dv))
    wantS = np.empty((len(lens), H, dk, dv))
    pos = 0
    for i, n in enumerate(lens):
        gam = np.cumsum(g[pos:pos + n].astype(np.float64), axis=0)  # [n, H]
        for h in range(H):
            S0 = h0[i, h].astype(np.float64)
            want[pos:pos + n, h] = np.exp(gam[:, h])[:, None] * (q[pos:pos + n, h].astype(np.float64) @ S0)
            wantS[i, h] = np.exp(gam[-1, h]) * S0
        pos += n
    err = float(np.max(np.abs(got - want)))
    assert err <= 1e-5 * float(np.max(np.abs(want))), err
    errS = float(np.max(np.abs(gotS - wantS)))
    assert errS <= 1e-5 * float(np.max(np.abs(wantS))), errS
