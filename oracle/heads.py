"""Key and query heads shared by groups of value heads, float64.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

The pages name hybrid Gated DeltaNet models (Chinese page, the paragraph
on the released code and the model classes it supports) but not their layer
dimensions; layers of that kind may give the queries and keys fewer heads
than the values.  Reading used here:
with H value heads and H_k key heads (H a multiple of H_k, G = H / H_k),
value head h reads the query and key of key head floor(h / G), so heads
jG .. jG + G - 1 share key head j; everything else (state, decay, beta,
value, output) belongs to the value head.  Written out as the definition:
the shared query and key rows are repeated once per value head, and the
gradient of a shared row is the sum of its group's gradients.
"""

from __future__ import annotations

import numpy as np


def group_size(num_heads: int, num_key_heads: int) -> int:
    if num_key_heads <= 0 or num_heads % num_key_heads != 0:
        raise ValueError(f"{num_heads} value heads cannot share {num_key_heads} key heads")
    return num_heads // num_key_heads


def expand_key_heads(x: np.ndarray, num_heads: int) -> np.ndarray:
    """[T, H_k, d] -> [T, H, d]: key head j repeated for value heads jG .. jG+G-1."""
    x = np.asarray(x, np.float64)
    G = group_size(num_heads, x.shape[1])
    return x if G == 1 else np.repeat(x, G, axis=1)


def sum_key_heads(dx: np.ndarray, num_key_heads: int) -> np.ndarray:
    """[T, H, d] -> [T, H_k, d]: sum over each group of value heads."""
    T, H, d = dx.shape
    G = group_size(H, num_key_heads)
    return dx if G == 1 else dx.reshape(T, num_key_heads, G, d).sum(axis=2)
