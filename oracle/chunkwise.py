"""Chunk (WY / UT-transform) form of the Gated DeltaNet layer in float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Written independently of recurrent.py and pinned against it.  The pages say
that training and prefill first compute the recurrent state at every chunk
boundary (Chinese page, section on the "third way" for Gated DeltaNet); this
module is the chunk algebra that produces those boundary states, plus the
chunk-form outputs that "native" chunkwise kernels would use.

Within one chunk of n tokens that starts from state B (M-form, d_v x d_k), with
local positions t = 1..n:
  gamma_t = sum_{s<=t} g_s,  Gamma_t = exp(gamma_t)
  D[t,s]  = exp(gamma_t - gamma_s) for s <= t, else 0
  e_s     = exp(gamma_n - gamma_s)
  G       = K K^T
  L       = strictly lower part of (beta_t D[t,s] G[t,s])
  T       = (I + L)^{-1} diag(beta)
  W       = T diag(Gamma) K          (n x d_k)
  U       = T V                      (n x d_v)
  Delta   = U - W B^T                (rows are the delta-rule corrections u_t)
  B'      = Gamma_n B + Delta^T diag(e) K
  O       = diag(Gamma) Q B^T + ((Q K^T) * D) Delta
Derivation: unrolling the recurrence inside the chunk gives
u_t = beta_t (v_t - Gamma_t B k_t - sum_{s<t} D[t,s] (k_s . k_t) u_s), i.e.
(I + L) Delta = diag(beta) (V - diag(Gamma) K B^T), and
M_t = Gamma_t B + sum_{s<=t} D[t,s] u_s k_s^T.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .heads import expand_key_heads


def chunk_products(K: np.ndarray, V: np.ndarray, g: np.ndarray, beta: np.ndarray):
    """Chunk-local products for one head: (W, U, Ktilde, Gamma_n, T, D, Gamma).

    K [n, d_k], V [n, d_v], g, beta [n], all float64.
    Ktilde = diag(e) K.
    """
    n = K.shape[0]
    gamma = np.cumsum(g)
    Gam = np.exp(gamma)
    diff = gamma[:, None] - gamma[None, :]
    lower_incl = np.tril(np.ones((n, n), dtype=bool))
    D = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
    G = K @ K.T
    L = np.tril(beta[:, None] * D * G, k=-1)
    T = np.linalg.solve(np.eye(n) + L, np.diag(beta))
    W = T @ (Gam[:, None] * K)
    U = T @ V
    e = np.exp(gamma[-1] - gamma) if n > 0 else np.zeros(0)
    Kt = e[:, None] * K
    Gn = Gam[-1] if n > 0 else 1.0
    return W, U, Kt, Gn, T, D, Gam


def chunkwise_forward(q, k, v, g, beta, cu_seqlens, h0: Optional[np.ndarray] = None,
                      chunk: int = 64, return_boundaries: bool = False):
    """Chunk-form forward over a packed varlen batch, float64.

    Chunks start at each sequence's first token; the last chunk of a sequence
    may be shorter than `chunk`.  Returns (o [T,H,d_v], hT [N,H,d_k,d_v]); with
    return_boundaries also a list (per sequence) of [n_chunks+1, H, d_k, d_v]
    boundary states (S layout), index 0 = initial state.
    """
    v = np.asarray(v, np.float64)
    q = expand_key_heads(q, v.shape[1])  # q, k may have fewer heads (heads.py)
    k = expand_key_heads(k, v.shape[1])
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    N = cu.shape[0] - 1
    T, H, dk = q.shape
    dv = v.shape[2]
    o = np.zeros((T, H, dv))
    hT = np.zeros((N, H, dk, dv))
    bounds = []
    for i in range(N):
        a, b = int(cu[i]), int(cu[i + 1])
        nchunks = (b - a + chunk - 1) // chunk
        bl = np.zeros((nchunks + 1, H, dk, dv))
        for h in range(H):
            B = np.zeros((dv, dk)) if h0 is None else np.asarray(h0[i, h], np.float64).T.copy()
            bl[0, h] = B.T
            for c in range(nchunks):
                s0 = a + c * chunk
                s1 = min(s0 + chunk, b)
                Q = q[s0:s1, h]
                K = k[s0:s1, h]
                V = v[s0:s1, h]
                W, U, Kt, Gn, _T, D, Gam = chunk_products(K, V, g[s0:s1, h], beta[s0:s1, h])
                Delta = U - W @ B.T
                o[s0:s1, h] = Gam[:, None] * (Q @ B.T) + ((Q @ K.T) * D) @ Delta
                B = Gn * B + Delta.T @ Kt
                bl[c + 1, h] = B.T
            hT[i, h] = B.T
        bounds.append(bl)
    if return_boundaries:
        return o, hT, bounds
    return o, hT
