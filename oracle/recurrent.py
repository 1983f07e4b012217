"""Token-by-token Gated DeltaNet recurrence in float64 (the definition).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Source of the update: the IsoExec pages describe CPR as keeping the recurrence
as the main function ("Chunkwise-Parallel Recurrent (CPR) Gated DeltaNet",
English page; same section on the Korean page); the recurrence is the Gated
DeltaNet update
    M_t = alpha_t M_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = M_t q_t,  alpha_t = exp(g_t),
with the output read after the update.  It is evaluated here as the
equivalent sequence
    M' = alpha M;  p = M' k;  u = beta (v - p);  M = M' + u k^T;  o = M q,
which tests/test_oracle.py checks against the literal matrix product form.

Sequences in a packed batch are independent; each starts from its own initial
state (zero when none is given).
"""

from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .heads import expand_key_heads


def token_step(M: np.ndarray, q: np.ndarray, k: np.ndarray, v: np.ndarray,
               g: np.ndarray, beta: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """One step for a batch of heads.

    M [B, d_v, d_k]; q, k [B, d_k]; v [B, d_v]; g, beta [B].
    Returns (new M, o [B, d_v]).
    """
    a = np.exp(g)[:, None, None]
    Mp = a * M
    p = np.einsum("bji,bi->bj", Mp, k)
    u = beta[:, None] * (v - p)
    Mn = Mp + u[:, :, None] * k[:, None, :]
    o = np.einsum("bji,bi->bj", Mn, q)
    return Mn, o


def recurrent_forward(q, k, v, g, beta, cu_seqlens, h0: Optional[np.ndarray] = None,
                      return_all_states: bool = False):
    """Run the recurrence over a packed varlen batch in float64.

    q, k [T, H_k, d_k] (H_k divides H; see heads.py); v [T, H, d_v];
    g, beta [T, H]; cu_seqlens [N+1]; h0 [N, H, d_k, d_v] or None.
    Returns (o [T, H, d_v] float64, hT [N, H, d_k, d_v] float64).
    If return_all_states, also a list (per sequence) of [L+1, H, d_v, d_k]
    M-form states (index 0 = initial state).
    """
    v = np.asarray(v, np.float64)
    q = expand_key_heads(q, v.shape[1])
    k = expand_key_heads(k, v.shape[1])
    g = np.asarray(g, np.float64)
    beta = np.asarray(beta, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    N = cu.shape[0] - 1
    T, H, dk = q.shape
    dv = v.shape[2]
    lengths = np.diff(cu)
    o = np.zeros((T, H, dv), np.float64)
    # M-form state per (sequence, head)
    if h0 is None:
        M = np.zeros((N, H, dv, dk), np.float64)
    else:
        M = np.ascontiguousarray(np.swapaxes(np.asarray(h0, np.float64), -1, -2))
    states = None
    if return_all_states:
        states = [np.zeros((int(lengths[i]) + 1, H, dv, dk)) for i in range(N)]
        for i in range(N):
            states[i][0] = M[i]
    max_len = int(lengths.max()) if N > 0 else 0
    # Sequences advance in lockstep over their local position t; a sequence
    # whose length is reached simply stops being updated.
    for t in range(max_len):
        act = np.nonzero(lengths > t)[0]
        rows = cu[act] + t
        Ma = M[act].reshape(-1, dv, dk)
        Mn, ot = token_step(Ma, q[rows].reshape(-1, dk), k[rows].reshape(-1, dk),
                            v[rows].reshape(-1, dv), g[rows].reshape(-1),
                            beta[rows].reshape(-1))
        M[act] = Mn.reshape(len(act), H, dv, dk)
        o[rows] = ot.reshape(len(act), H, dv)
        if states is not None:
            for j, i in enumerate(act):
                states[i][t + 1] = M[i]
    hT = np.ascontiguousarray(np.swapaxes(M, -1, -2))
    if return_all_states:
        return o, hT, states
    return o, hT
