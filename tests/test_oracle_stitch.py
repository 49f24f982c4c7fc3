"""Pins for the oracle's tile stitching."""

import numpy as np

from oracle import mds, stitch
from workloads import packed_distances, random_walk, walk_rng


def _random_orthogonal(rng, reflect):
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if reflect:
        q[:, 0] *= -1
    return q


def _tiles(chain, L, n=64, O=12):
    stride = n - O
    return np.stack([chain[k * stride:k * stride + n] for k in range(L)])


def test_stitch_undoes_per_tile_rigid_motions():
    rng = np.random.default_rng(1)
    L, O = 6, 12
    chain = random_walk((L - 1) * 52 + 64, walk_rng(3, 1), None)
    tiles = _tiles(chain, L)
    moved = np.stack([t @ _random_orthogonal(rng, k % 2 == 1) + rng.standard_normal(3) * 10
                      for k, t in enumerate(tiles)])
    got, resid = stitch.stitch_chain(moved, O)
    assert got.shape == chain.shape
    assert np.all(resid < 1e-9)
    # the stitched chain is the original up to tile 0's motion: every distance is reproduced
    assert np.allclose(packed_distances(got), packed_distances(chain), atol=1e-9, rtol=0)


def test_residual_equals_brute_force_rms_after_alignment():
    rng = np.random.default_rng(2)
    tiles = rng.standard_normal((3, 64, 3)) * 5
    got, resid = stitch.stitch_chain(tiles, 12)
    # the alignment is optimal: no random orthogonal map does better on seam 0
    x, y = tiles[1][:12], tiles[0][52:]
    best = resid[0]
    for _ in range(200):
        q = _random_orthogonal(rng, rng.integers(2) == 1)
        xm, ym = x.mean(0), y.mean(0)
        d = (x - xm) @ q + ym - y
        assert np.sqrt(np.mean(np.sum(d * d, axis=1))) >= best - 1e-12
    # shared beads hold the mean of both aligned copies: bead 52 of tile 0 is global bead 52
    r, shift = stitch.align(x, y)
    assert np.allclose(got[52], 0.5 * (tiles[0][52] + tiles[1][0] @ r + shift))


def test_stitch_after_mds_of_each_tile():
    # MDS of each tile's exact map gives each tile in its own frame; stitching restores the chain
    L = 4
    chain = random_walk((L - 1) * 52 + 64, walk_rng(5, 2), None)
    tiles = _tiles(chain, L)
    rec = np.stack([mds.classical_mds(packed_distances(t))[0] for t in tiles])
    got, resid = stitch.stitch_chain(rec, 12)
    assert np.all(resid < 1e-8)
    assert np.allclose(packed_distances(got), packed_distances(chain), atol=1e-8, rtol=0)
