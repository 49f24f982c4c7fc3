"""Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
1, 2, 3", SC'11) — oracle implementation, test infrastructure.

A Philox-4x32 round takes a 4-word counter (c0, c1, c2, c3) and a 2-word key
(k0, k1), forms the two 64-bit products M0*c0 and M1*c2, and returns

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0)).

Between rounds the key is bumped by the Weyl constants (W0, W1) modulo 2^32.
Ten rounds make one block.  The multipliers and Weyl constants are the
published Philox-4x32 parameters.

Keying used by the sampler: key = (seed mod 2^32, seed >> 32); counter =
(quad q of the map, trajectory id t, step slot, 0).  Slot 0 draws x_T; slot
i + 1 draws the noise of DDIM step i.  Word l of block q belongs to packed
element 4q + l.

Two implementations: ``block`` on Python integers (scalar, the plain
definition) and ``blocks`` on numpy uint64 arrays (vectorised).
"""

from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
ROUNDS = 10
MASK32 = 0xFFFFFFFF


def key_from_seed(seed: int) -> tuple[int, int]:
    return seed & MASK32, (seed >> 32) & MASK32


def block(counter, key) -> tuple[int, int, int, int]:
    """One Philox4x32-10 block on Python integers."""
    c0, c1, c2, c3 = (int(v) & MASK32 for v in counter)
    k0, k1 = (int(v) & MASK32 for v in key)
    for r in range(ROUNDS):
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0, p1 & MASK32, (p0 >> 32) ^ c3 ^ k1, p0 & MASK32)
        if r != ROUNDS - 1:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
    return c0, c1, c2, c3


def blocks(c0, c1, c2, c3, key) -> np.ndarray:
    """Vectorised Philox4x32-10.  Counters broadcast against each other.

    Returns uint32 [..., 4] with the four output words of each block.
    """
    b = np.broadcast(c0, c1, c2, c3)
    x0, x1, x2, x3 = (np.broadcast_to(np.asarray(v, dtype=np.uint64), b.shape) & np.uint64(MASK32)
                      for v in (c0, c1, c2, c3))
    k0, k1 = key
    m32 = np.uint64(MASK32)
    sh = np.uint64(32)
    for r in range(ROUNDS):
        p0 = np.uint64(M0) * x0
        p1 = np.uint64(M1) * x2
        x0, x1, x2, x3 = ((p1 >> sh) ^ x1 ^ np.uint64(k0), p1 & m32, (p0 >> sh) ^ x3 ^ np.uint64(k1), p0 & m32)
        if r != ROUNDS - 1:
            k0 = (k0 + W0) & MASK32
            k1 = (k1 + W1) & MASK32
    return np.stack([x0, x1, x2, x3], axis=-1).astype(np.uint32)


def map_words(seed: int, traj_ids, slot: int, n_packed: int = 2016) -> np.ndarray:
    """uint32 [len(traj_ids), n_packed]: the Philox word for every packed element.

    Element e of trajectory t takes word e % 4 of the block with counter
    (e // 4, t, slot, 0).
    """
    if n_packed % 4:
        raise ValueError("packed length must be a multiple of 4")
    t = np.asarray(traj_ids, dtype=np.uint64).reshape(-1, 1)
    q = np.arange(n_packed // 4, dtype=np.uint64).reshape(1, -1)
    w = blocks(q, t, np.uint64(slot), np.uint64(0), key_from_seed(seed))
    return w.reshape(t.shape[0], n_packed)
