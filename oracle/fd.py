"""Central finite differences of the layer's scalar loss, float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Loss: L = sum(o * dO) + sum(S_T * dhT), with (o, S_T) from the token
recurrence.  Used only to pin the analytic backward on tiny instances.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .recurrent import recurrent_forward


def loss_value(inputs: dict, cu_seqlens, d_o, d_hT: Optional[np.ndarray]) -> float:
    o, hT = recurrent_forward(inputs["q"], inputs["k"], inputs["v"], inputs["g"],
                              inputs["beta"], cu_seqlens, inputs.get("h0"))
    val = float(np.sum(o * d_o))
    if d_hT is not None:
        val += float(np.sum(hT * d_hT))
    return val


def fd_gradients(inputs: dict, cu_seqlens, d_o, d_hT=None, h: float = 1e-6,
                 names=("q", "k", "v", "g", "beta", "h0")) -> dict:
    """Central differences (L(x+h) - L(x-h)) / 2h for every entry of each input."""
    base = {n: np.array(a, dtype=np.float64, copy=True) for n, a in inputs.items() if a is not None}
    out = {}
    for name in names:
        if name not in base:
            continue
        x = base[name]
        grad = np.zeros_like(x)
        flat = x.reshape(-1)
        gflat = grad.reshape(-1)
        for j in range(flat.size):
            old = flat[j]
            flat[j] = old + h
            lp = loss_value(base, cu_seqlens, d_o, d_hT)
            flat[j] = old - h
            lm = loss_value(base, cu_seqlens, d_o, d_hT)
            flat[j] = old
            gflat[j] = (lp - lm) / (2.0 * h)
        out[name] = grad
    return out
