"""Seeded synthetic inputs for a Gated DeltaNet layer.

This module is shared by the CPU oracle and by the HIP path's tests and
benchmark.  It holds none of the layer's arithmetic: it only draws random
numbers with the distributions used for every workload and rounds them to the
storage dtype.

Distributions (per token t and head h):
  q, k  ~ N(0, 1), then divided by their L2 norm over the key dimension (fp32)
  v     ~ N(0, 1)
  beta  = sigmoid(z),            z ~ N(0, 1)
  g     = -softplus(z) * 0.1,    z ~ N(0, 1)   (so alpha = exp(g) is about 0.93)
  h0    ~ N(0, h0_std) per state entry, when an initial state is requested
  dO    ~ N(0, 1), when an upstream output gradient is requested
For bf16 workloads every tensor except h0 is rounded to bf16 (round to
nearest, ties to even) after it is drawn; the fp32 arrays returned then hold
exactly the bf16 values, so the GPU path (fed the bf16 bits) and the oracle
(fed the same values as fp64) consume identical numbers.

Reproducibility: sequence lengths come from a generator seeded with
(seed, 0); sequence i draws its own tensors from a generator seeded with
(seed, i + 1), in the fixed order q, k, v, beta-logit, g-logit, h0, dO.  So a
sequence's values do not depend on which other sequences share its batch.

Layouts (packed varlen batch of N sequences, T tokens in total):
  q, k [T, H_k, d_k] (H_k = H unless fewer key heads are asked for; H_k
  divides H); v, dO [T, H, d_v]; g, beta [T, H];
  cu_seqlens int32 [N + 1]; h0 [N, H, d_k, d_v] (the state S = M^T, key
  dimension first).
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Batch",
    "round_to_bf16",
    "bf16_bits",
    "from_bf16_bits",
    "draw_lengths",
    "make_batch",
    "workload",
    "WORKLOADS",
]


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value (ties to even); returns fp32.

    Only finite inputs are expected (the distributions above are finite).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns of fp32 values that are already bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("values are not exactly representable in bf16")
    return (u >> np.uint32(16)).astype(np.uint16)


def from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """fp32 values of uint16 bf16 bit patterns (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Batch:
    """A packed varlen batch.  Float arrays are fp32 holding dtype-exact values."""

    dtype: str  # "f32" or "bf16"
    num_heads: int
    d_k: int
    d_v: int
    cu_seqlens: np.ndarray  # int32 [N+1]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    h0: Optional[np.ndarray] = None  # fp32 [N,H,d_k,d_v] or None (zero state)
    d_o: Optional[np.ndarray] = None  # [T,H,d_v] or None
    num_key_heads: int = 0  # heads of q and k (0: num_heads)

    def __post_init__(self):
        if self.num_key_heads == 0:
            self.num_key_heads = self.num_heads

    @property
    def num_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens).astype(np.int64)

    def seq_slice(self, i: int) -> slice:
        return slice(int(self.cu_seqlens[i]), int(self.cu_seqlens[i + 1]))

    def select(self, seqs: Sequence[int]) -> "Batch":
        """A new packed batch holding only the given sequences, in that order."""
        seqs = list(seqs)
        parts = [self.seq_slice(i) for i in seqs]
        lens = [p.stop - p.start for p in parts]
        cu = np.zeros(len(seqs) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)

        def cat(a):
            if a is None:
                return None
            if not parts:
                return a[:0].copy()
            return np.ascontiguousarray(np.concatenate([a[p] for p in parts], axis=0))

        h0 = None if self.h0 is None else np.ascontiguousarray(self.h0[seqs])
        return Batch(self.dtype, self.num_heads, self.d_k, self.d_v, cu,
                     cat(self.q), cat(self.k), cat(self.v), cat(self.g), cat(self.beta),
                     h0, cat(self.d_o), self.num_key_heads)

    def truncate(self, lengths: Sequence[int]) -> "Batch":
        """Keep the first lengths[i] tokens of every sequence i."""
        lens = [int(x) for x in lengths]
        own = self.lengths
        if len(lens) != self.num_seqs or any(a > b or a < 0 for a, b in zip(lens, own)):
            raise ValueError("bad truncation lengths")
        idx = np.concatenate([np.arange(int(self.cu_seqlens[i]), int(self.cu_seqlens[i]) + n)
                              for i, n in enumerate(lens)]) if lens else np.zeros(0, np.int64)
        cu = np.zeros(len(lens) + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)

        def take(a):
            return None if a is None else np.ascontiguousarray(a[idx])

        return Batch(self.dtype, self.num_heads, self.d_k, self.d_v, cu,
                     take(self.q), take(self.k), take(self.v), take(self.g), take(self.beta),
                     None if self.h0 is None else self.h0.copy(), take(self.d_o), self.num_key_heads)


def draw_lengths(seed: int, num_seqs: int, low: int, high: int) -> np.ndarray:
    """Sequence lengths uniform in [low, high] from the (seed, 0) stream."""
    rng = np.random.default_rng([seed, 0])
    return rng.integers(low, high + 1, size=num_seqs).astype(np.int64)


def _unit_rows(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True, dtype=np.float32))
    return (x / n).astype(np.float32)


def make_batch(seed: int, lengths: Sequence[int], num_heads: int, d_k: int, d_v: int,
               dtype: str = "bf16", h0_std: Optional[float] = None,
               with_do: bool = False, num_key_heads: Optional[int] = None) -> Batch:
    """Draw a packed batch; sequence i uses the (seed, i + 1) stream.

    num_key_heads: heads of q and k (default num_heads; must divide it)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    lengths = [int(n) for n in lengths]
    H = num_heads
    Hk = H if num_key_heads is None else int(num_key_heads)
    if Hk <= 0 or H % Hk != 0:
        raise ValueError("num_key_heads must divide num_heads")
    T = int(sum(lengths))
    q = np.empty((T, Hk, d_k), np.float32)
    k = np.empty((T, Hk, d_k), np.float32)
    v = np.empty((T, H, d_v), np.float32)
    g = np.empty((T, H), np.float32)
    beta = np.empty((T, H), np.float32)
    d_o = np.empty((T, H, d_v), np.float32) if with_do else None
    h0 = np.empty((len(lengths), H, d_k, d_v), np.float32) if h0_std is not None else None
    rnd = round_to_bf16 if dtype == "bf16" else (lambda a: a.astype(np.float32))
    pos = 0
    for i, n in enumerate(lengths):
        rng = np.random.default_rng([seed, i + 1])
        sl = slice(pos, pos + n)
        q[sl] = rnd(_unit_rows(rng.standard_normal((n, Hk, d_k), dtype=np.float32)))
        k[sl] = rnd(_unit_rows(rng.standard_normal((n, Hk, d_k), dtype=np.float32)))
        v[sl] = rnd(rng.standard_normal((n, H, d_v), dtype=np.float32))
        zb = rng.standard_normal((n, H), dtype=np.float32)
        beta[sl] = rnd((1.0 / (1.0 + np.exp(-zb.astype(np.float64)))).astype(np.float32))
        zg = rng.standard_normal((n, H), dtype=np.float32)
        g[sl] = rnd((-np.logaddexp(0.0, zg.astype(np.float64)) * 0.1).astype(np.float32))
        if h0 is not None:
            h0[i] = (rng.standard_normal((H, d_k, d_v), dtype=np.float32) * np.float32(h0_std))
        if d_o is not None:
            d_o[sl] = rnd(rng.standard_normal((n, H, d_v), dtype=np.float32))
        pos += n
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return Batch(dtype, H, d_k, d_v, cu, q, k, v, g, beta, h0, d_o, Hk)


# The five workloads the layer is exercised on.  Each entry: seed, sequence
# lengths (prefill part), decode tokens per sequence after the prefill, heads,
# head dims, chunk size, dtype, initial-state std (None = zero state), whether
# an upstream gradient is drawn.
WORKLOADS = {
    # tiny fp32 forward: prefill, then the same tokens one by one through decode
    "tiny_f32": dict(seed=1, num_seqs=1, prefill_len=256, decode_len=0, H=2, d=64, C=64,
                     dtype="f32", h0_std=None, with_do=False),
    # prefill 5 x 2,048 tokens
    "prefill_5x2048": dict(seed=2, num_seqs=5, prefill_len=2048, decode_len=0, H=16, d=128,
                           C=64, dtype="bf16", h0_std=None, with_do=False),
    # decode: 256 sequences, 2,048-token prefix then 128 single-token steps
    "decode_256x1": dict(seed=3, num_seqs=256, prefill_len=2048, decode_len=128, H=16,
                         d=128, C=64, dtype="bf16", h0_std=None, with_do=False),
    # trainer forward + backward, 1 x 10,240 tokens
    "train_1x10240": dict(seed=4, num_seqs=1, prefill_len=10240, decode_len=0, H=16, d=128,
                          C=64, dtype="bf16", h0_std=None, with_do=True),
    # varlen packed batch: 64 sequences, lengths U[1, 8192], then 100 decode steps
    "varlen_64": dict(seed=5, num_seqs=64, prefill_len=(1, 8192), decode_len=100, H=32,
                      d=128, C=64, dtype="bf16", h0_std=0.1, with_do=False),
}


def workload(name: str, num_seqs: Optional[int] = None, heads: Optional[int] = None):
    """(Batch holding prefill + decode tokens, prefill lengths, decode_len, C).

    num_seqs / heads optionally shrink the workload (keeping the first
    sequences' values, since every sequence has its own stream).
    """
    w = WORKLOADS[name]
    n = w["num_seqs"] if num_seqs is None else int(num_seqs)
    if isinstance(w["prefill_len"], tuple):
        lo, hi = w["prefill_len"]
        pre = draw_lengths(w["seed"], w["num_seqs"], lo, hi)[:n]
    else:
        pre = np.full(n, w["prefill_len"], dtype=np.int64)
    H = w["H"] if heads is None else int(heads)
    total = pre + w["decode_len"]
    b = make_batch(w["seed"], total, H, w["d"], w["d"], w["dtype"], w["h0_std"], w["with_do"])
    return b, pre, w["decode_len"], w["C"]
