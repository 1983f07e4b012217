"""Analytic reverse-mode gradient of the Gated DeltaNet recurrence, float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages give the trainer forward+backward only as a timing (English page,
CPR table; Chinese page, "third way" section); any exact gradient of the
recurrence is correct.  This is the token-level reverse pass of the forward in
recurrent.py.  For the scalar loss
    L = sum_t <dO_t, o_t> + sum_seq <dhT, S_T>
and each token step (M' = a M_prev, p = M' k, u = beta (v - p),
M = M' + u k^T, o = M q, a = exp(g)), going backwards with dM = dL/dM_t:
    dM += dO_t q^T;      dq_t  = M^T dO_t
    du  = dM k;          dk_t  = dM^T u
    dbeta_t = <du, v - p>;  dv_t = beta du;  dp = -beta du
    dM' = dM + dp k^T;   dk_t += M'^T dp
    dg_t = a <dM', M_prev>
    dM_prev = a dM'
and finally dh0 = dM.  States inside a sequence are recomputed from the saved
initial state (the whole trajectory is kept for the short sequences the tests
use; `checkpoint` chunks bound the memory for long ones).
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .heads import expand_key_heads, sum_key_heads
from .recurrent import token_step


def recurrent_backward(q, k, v, g, beta, cu_seqlens, h0: Optional[np.ndarray],
                       d_o: np.ndarray, d_hT: Optional[np.ndarray] = None,
                       checkpoint: int = 64):
    """Gradients of L w.r.t. (q, k, v, g, beta, h0).

    Returns dict with dq, dk [T,H_k,d_k] (the shapes of q, k; a key head
    shared by several value heads receives the sum of their gradients, see
    heads.py); dv [T,H,d_v]; dg, dbeta [T,H]; dh0 [N,H,d_k,d_v] (S layout);
    all float64.
    """
    v = np.asarray(v, np.float64)
    num_key_heads = np.asarray(q).shape[1]
    q = expand_key_heads(q, v.shape[1])
    k = expand_key_heads(k, v.shape[1])
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    d_o = np.asarray(d_o, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    N = cu.shape[0] - 1
    T, H, dk = q.shape
    dv = v.shape[2]
    dq = np.zeros((T, H, dk))
    dkk = np.zeros((T, H, dk))
    dvv = np.zeros((T, H, dv))
    dg = np.zeros((T, H))
    db = np.zeros((T, H))
    dh0 = np.zeros((N, H, dk, dv))
    for i in range(N):
        a0, b0 = int(cu[i]), int(cu[i + 1])
        n = b0 - a0
        M = np.zeros((H, dv, dk)) if h0 is None else np.swapaxes(np.asarray(h0[i], np.float64), -1, -2).copy()
        # forward pass keeping the state at every checkpoint
        ckpt = {0: M.copy()}
        for t in range(n):
            r = a0 + t
            M, _ = token_step(M, q[r], k[r], v[r], g[r], beta[r])
            if (t + 1) % checkpoint == 0:
                ckpt[t + 1] = M.copy()
        dM = np.zeros((H, dv, dk)) if d_hT is None else np.swapaxes(np.asarray(d_hT[i], np.float64), -1, -2).copy()
        # reverse over checkpoint segments
        seg_starts = sorted(ckpt.keys())
        for s0 in reversed(seg_starts):
            s1 = min(s0 + checkpoint, n)
            if s1 <= s0:
                continue
            states = [ckpt[s0]]
            Mc = ckpt[s0]
            for t in range(s0, s1):
                Mc, _ = token_step(Mc, q[a0 + t], k[a0 + t], v[a0 + t], g[a0 + t], beta[a0 + t])
                states.append(Mc)
            for t in range(s1 - 1, s0 - 1, -1):
                r = a0 + t
                Mprev = states[t - s0]
                Mt = states[t - s0 + 1]
                a = np.exp(g[r])  # [H]
                Mp = a[:, None, None] * Mprev
                kt, qt, vt, bt = k[r], q[r], v[r], beta[r]
                p = np.einsum("hji,hi->hj", Mp, kt)
                u = bt[:, None] * (vt - p)
                dot = d_o[r]
                dM = dM + dot[:, :, None] * qt[:, None, :]
                dq[r] = np.einsum("hji,hj->hi", Mt, dot)
                du = np.einsum("hji,hi->hj", dM, kt)
                dk_t = np.einsum("hji,hj->hi", dM, u)
                db[r] = np.sum(du * (vt - p), axis=1)
                dvv[r] = bt[:, None] * du
                dp = -bt[:, None] * du
                dMp = dM + dp[:, :, None] * kt[:, None, :]
                dk_t = dk_t + np.einsum("hji,hj->hi", Mp, dp)
                dkk[r] = dk_t
                dg[r] = a * np.sum(dMp * Mprev, axis=(1, 2))
                dM = a[:, None, None] * dMp
        dh0[i] = np.swapaxes(dM, -1, -2)
    return dict(dq=sum_key_heads(dq, num_key_heads), dk=sum_key_heads(dkk, num_key_heads), dv=dvv, dg=dg,
                dbeta=db, dh0=dh0)
