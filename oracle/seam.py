"""Overlap-consistency projection and seam discrepancy — oracle, test infrastructure.

Tiling (ParaChromo, sections 3.2 and 4.3): adjacent 64-bead tiles share O
beads (O = 12); the lower-right O x O block of the left tile's map and the
upper-left O x O block of the right tile's map describe the same monomer
pairs.  Seam k joins tile k (local beads 64-O .. 63) with tile k+1 (local
beads 0 .. O-1).  In the packed layout the seam holds O(O-1)/2 distinct pairs
(66 for O = 12): pair (p, q), p < q < O, sits at idx(64-O+p, 64-O+q) in tile k
and at idx(p, q) in tile k+1.

Projection (ParaChromo, section 4.3.2 and Algorithm 1): for every adjacent
pair of tiles and every batch index b (the same b across tiles is one joint
tiled sample), both copies of each shared pair are replaced by their mean.
Only seam entries change; symmetry is kept because only the packed upper
triangle is stored.

Discrepancy: per (seam, b), the root-mean-square difference of the two
copies over the shared pairs.  ``discrepancy_mean_abs`` is the paper's
Eq. (6) reading (section 5.5): the mean over shared pairs of the absolute
difference between the sample-mean overlap blocks of the two tiles.

States are float64 arrays [L, B, P]: L tiles of one chain, B joint samples.
"""

from __future__ import annotations

import numpy as np

from .layout import idx


def seam_pairs(overlap: int, n: int = 64):
    """(left_tile_idx, right_tile_idx) int64 arrays, pairs in (p, q) row-major order."""
    if not 1 <= overlap <= n // 2:
        raise ValueError("overlap out of range")
    off = n - overlap
    left, right = [], []
    for p in range(overlap):
        for q in range(p + 1, overlap):
            left.append(idx(off + p, off + q, n))
            right.append(idx(p, q, n))
    return np.array(left, dtype=np.int64), np.array(right, dtype=np.int64)


def project(states, overlap: int) -> np.ndarray:
    """Return a projected copy of a chain's states [L, B, P]."""
    x = np.array(states, dtype=np.float64, copy=True)
    li, ri = seam_pairs(overlap)
    for k in range(x.shape[0] - 1):
        m = (x[k][:, li] + x[k + 1][:, ri]) / 2.0
        x[k][:, li] = m
        x[k + 1][:, ri] = m
    return x


def discrepancy_rms(states, overlap: int) -> np.ndarray:
    """[L-1, B] RMS over the shared pairs of (left copy - right copy)."""
    x = np.asarray(states, dtype=np.float64)
    li, ri = seam_pairs(overlap)
    out = np.empty((x.shape[0] - 1, x.shape[1]))
    for k in range(x.shape[0] - 1):
        d = x[k][:, li] - x[k + 1][:, ri]
        out[k] = np.sqrt(np.mean(d * d, axis=1))
    return out


def discrepancy_mean_abs(states, overlap: int) -> np.ndarray:
    """[L-1] mean over shared pairs of |mean_b left copy - mean_b right copy|."""
    x = np.asarray(states, dtype=np.float64)
    li, ri = seam_pairs(overlap)
    out = np.empty(x.shape[0] - 1)
    for k in range(x.shape[0] - 1):
        out[k] = np.mean(np.abs(x[k][:, li].mean(axis=0) - x[k + 1][:, ri].mean(axis=0)))
    return out
