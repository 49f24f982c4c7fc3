"""Packed distance-map layout — oracle, test infrastructure.

A map of n beads stores the n(n-1)/2 distances of pairs i < j (the diagonal
is zero and the lower triangle mirrors the upper, so neither is stored), row
by row:  idx(i, j) = i (2n - i - 1) / 2 + (j - i - 1).
"""

from __future__ import annotations

from functools import lru_cache

import numpy as np


def n_packed(n: int) -> int:
    return n * (n - 1) // 2


def idx(i: int, j: int, n: int = 64) -> int:
    if not 0 <= i < j < n:
        raise ValueError("need 0 <= i < j < n")
    return i * (2 * n - i - 1) // 2 + (j - i - 1)


@lru_cache(maxsize=None)
def pair_table(n: int = 64):
    """(rows, cols): int arrays with rows[idx(i, j)] = i and cols[idx(i, j)] = j."""
    rows = np.empty(n_packed(n), dtype=np.int64)
    cols = np.empty(n_packed(n), dtype=np.int64)
    for i in range(n):
        for j in range(i + 1, n):
            rows[idx(i, j, n)] = i
            cols[idx(i, j, n)] = j
    rows.setflags(write=False)
    cols.setflags(write=False)
    return rows, cols


def unpack(x, n: int = 64) -> np.ndarray:
    """Packed [..., n(n-1)/2] -> symmetric [..., n, n] with a zero diagonal (float64)."""
    x = np.asarray(x, dtype=np.float64)
    rows, cols = pair_table(n)
    out = np.zeros(x.shape[:-1] + (n, n))
    out[..., rows, cols] = x
    out[..., cols, rows] = x
    return out


def pack(d, n: int = 64) -> np.ndarray:
    """Symmetric [..., n, n] -> packed strict upper triangle [..., n(n-1)/2]."""
    d = np.asarray(d, dtype=np.float64)
    rows, cols = pair_table(n)
    return d[..., rows, cols].copy()
