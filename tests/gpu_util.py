"""Helpers for the GPU tests: move seeded batches to the device and drive the
library through its C ABI (via the thin binding)."""

from __future__ import annotations

import sys

import numpy as np
import torch

import bitwise_invariant_gated_amd as gdn
from gdn_synth import Batch

DEV = "cuda"


def note(msg: str) -> None:
    """Name the case about to run on the GPU (flushed, so it survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def torch_dtype(b: Batch):
    return torch.bfloat16 if b.dtype == "bf16" else torch.float32


def shape_of(b: Batch, C: int = 64) -> gdn.LayerShape:
    return gdn.LayerShape(b.num_heads, b.d_k, b.d_v, C, torch_dtype(b), b.num_key_heads)


class DevBatch:
    def __init__(self, b: Batch, C: int = 64):
        dt = torch_dtype(b)
        self.b = b
        self.shape = shape_of(b, C)

        def t(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(DEV).to(dt).contiguous()

        self.q, self.k, self.v = t(b.q), t(b.k), t(b.v)
        self.g, self.beta = t(b.g), t(b.beta)
        self.cu = torch.from_numpy(b.cu_seqlens.astype(np.int32)).to(DEV)
        self.h0 = None if b.h0 is None else torch.from_numpy(b.h0).to(DEV).contiguous()
        self.d_o = None if b.d_o is None else t(b.d_o)


def prefill(db: DevBatch, cache=None, h0="batch"):
    b = db.b
    N, T = b.num_seqs, b.total_tokens
    if cache is None:
        cache = gdn.alloc_cache(db.shape, N)
    o = torch.empty((T, b.num_heads, b.d_v), dtype=torch_dtype(b), device=DEV)
    ws = gdn.alloc_workspace(db.shape, N, T, gdn.GDN_OP_PREFILL)
    gdn.gdn_cpr_prefill(db.shape, db.q, db.k, db.v, db.g, db.beta, db.cu,
                        db.h0 if h0 == "batch" else h0, cache, o, ws)
    return o, cache


def decode_rows(db: DevBatch, start: np.ndarray, steps: int, cache):
    """Decode `steps` tokens per sequence: sequence i's step s is packed row
    cu[i] + start[i] + s.  Returns o [steps, N, H, d_v]."""
    b = db.b
    N = b.num_seqs
    ws = gdn.alloc_workspace(db.shape, N, 0, gdn.GDN_OP_DECODE)
    outs = torch.empty((steps, N, b.num_heads, b.d_v), dtype=torch_dtype(b), device=DEV)
    base = torch.from_numpy((b.cu_seqlens[:-1].astype(np.int64) + np.asarray(start, np.int64))).to(DEV)
    for s in range(steps):
        rows = base + s
        q, k, v = db.q[rows].contiguous(), db.k[rows].contiguous(), db.v[rows].contiguous()
        g, beta = db.g[rows].contiguous(), db.beta[rows].contiguous()
        gdn.gdn_cpr_decode_step(db.shape, q, k, v, g, beta, cache, outs[s], ws)
    return outs


def state_of(shape: gdn.LayerShape, cache) -> torch.Tensor:
    """The state after each cached sequence's last token, exp(run_log_scale) * s_run,
    written out by the library (gdn_cpr_cache_state)."""
    return gdn.gdn_cpr_cache_state(shape, cache)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns (for bit-exact comparisons; -0.0 != +0.0, NaN == NaN)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy()
    return t.numpy()


def as_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def tol_for(b: Batch, ref_max: float) -> float:
    """fp32 inputs: 1e-5 relative to max|o|; bf16 inputs: 2e-2 absolute."""
    return 1e-5 * ref_max if b.dtype == "f32" else 2e-2
