"""Uniform and Gaussian variates from Philox words — oracle, test infrastructure.

Box-Muller (Box & Muller, 1958): for u1 in (0, 1] and u2 in [0, 1),
    z1 = sqrt(-2 ln u1) cos(2 pi u2),   z2 = sqrt(-2 ln u1) sin(2 pi u2)
are independent N(0, 1).

Uniforms take the top 24 bits of a 32-bit word, so they are exact in both
float32 and float64:  u1 = ((r >> 8) + 1) * 2^-24 in (0, 1],
u2 = (r >> 8) * 2^-24 in [0, 1).  Words (r0, r1) of a Philox block give the
normals of elements 4q and 4q+1 (cosine, then sine); words (r2, r3) give
elements 4q+2 and 4q+3.
"""

from __future__ import annotations

import numpy as np

TWO_M24 = 2.0 ** -24


def uniform_open0(words) -> np.ndarray:
    """(0, 1]: ((r >> 8) + 1) * 2^-24."""
    return ((np.asarray(words, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) + 1.0) * TWO_M24


def uniform_open1(words) -> np.ndarray:
    """[0, 1): (r >> 8) * 2^-24."""
    return (np.asarray(words, dtype=np.uint64) >> np.uint64(8)).astype(np.float64) * TWO_M24


def box_muller(u1, u2):
    rad = np.sqrt(-2.0 * np.log(u1))
    ang = 2.0 * np.pi * u2
    return rad * np.cos(ang), rad * np.sin(ang)


def words_to_normals(words) -> np.ndarray:
    """Map Philox words [..., 4k] (grouped in blocks of 4) to normals of the same shape."""
    w = np.asarray(words)
    if w.shape[-1] % 4:
        raise ValueError("last axis must hold whole Philox blocks")
    blk = w.reshape(*w.shape[:-1], -1, 4)
    out = np.empty(blk.shape, dtype=np.float64)
    for a, b in ((0, 1), (2, 3)):
        z_cos, z_sin = box_muller(uniform_open0(blk[..., a]), uniform_open1(blk[..., b]))
        out[..., a] = z_cos
        out[..., b] = z_sin
    return out.reshape(w.shape)
