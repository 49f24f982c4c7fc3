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


def _random_rotation(rng):
    q = _random_orthogonal(rng, False)
    if np.linalg.det(q) < 0:
        q[:, 0] *= -1
    return q


def _rms_after(x, y, r):
    xm, ym = x.mean(0), y.mean(0)
    d = (x - xm) @ r + ym - y
    return np.sqrt(np.mean(np.sum(d * d, axis=1)))


def test_proper_fit_is_the_best_rotation():
    """Kabsch restricted to rotations: det +1; where the best orthogonal map is a
    reflection, no random rotation beats the fit, and its sum of squares exceeds the
    orthogonal optimum by exactly 4 sigma_3 (the objective is |X|^2 + |Y|^2 - 2 tr(R^T H),
    maximal over O(3) at sigma_1 + sigma_2 + sigma_3 and over SO(3) at sigma_1 + sigma_2 -
    sigma_3 when det(U V^T) = -1)."""
    rng = np.random.default_rng(11)
    n_reflected = 0
    for trial in range(20):
        x = rng.standard_normal((12, 3)) * 3
        m = _random_rotation(rng) @ (np.diag([1.0, 1.0, -1.0]) if trial % 2 else np.eye(3))
        y = x @ m + rng.standard_normal(3) + rng.standard_normal((12, 3)) * 0.3
        r, shift = stitch.align(x, y, proper=True)
        assert abs(np.linalg.det(r) - 1.0) < 1e-12
        assert np.allclose(r.T @ r, np.eye(3), atol=1e-12)
        ro, _ = stitch.align(x, y)
        xc, yc = x - x.mean(0), y - y.mean(0)
        sig = np.linalg.svd(xc.T @ yc, compute_uv=False)
        sse_p = 12 * _rms_after(x, y, r) ** 2
        sse_o = 12 * _rms_after(x, y, ro) ** 2
        if np.linalg.det(ro) < 0:
            n_reflected += 1
            assert np.isclose(sse_p, sse_o + 4 * sig[2], rtol=1e-10, atol=1e-10)
        else:
            assert np.allclose(r, ro, atol=1e-12)
        best = _rms_after(x, y, r)
        for _ in range(100):
            q = _random_rotation(rng)
            assert _rms_after(x, y, q) >= best - 1e-12
        assert np.allclose(shift, y.mean(0) - x.mean(0) @ r)
    assert n_reflected >= 5


def test_proper_stitching_undoes_rotations_and_keeps_mirrored_tiles_apart():
    rng = np.random.default_rng(4)
    L, O = 5, 12
    chain = random_walk((L - 1) * 52 + 64, walk_rng(9, 1), None)
    tiles = _tiles(chain, L)
    rotated = np.stack([t @ _random_rotation(rng) + rng.standard_normal(3) * 10 for t in tiles])
    got, resid = stitch.stitch_chain(rotated, O, proper=True)
    assert np.all(resid < 1e-9)
    assert np.allclose(packed_distances(got), packed_distances(chain), atol=1e-9, rtol=0)
    # a mirrored tile cannot be superposed by a rotation: its seams keep a residual of the
    # order of the overlap block's size, while the orthogonal fit closes them
    mirrored = rotated.copy()
    mirrored[2] = mirrored[2] @ np.diag([1.0, 1.0, -1.0])
    _, res_p = stitch.stitch_chain(mirrored, O, proper=True)
    _, res_o = stitch.stitch_chain(mirrored, O)
    assert np.all(res_o < 1e-9)
    assert res_p[1] > 0.1 and res_p[0] < 1e-9 and res_p[3] < 1e-9
