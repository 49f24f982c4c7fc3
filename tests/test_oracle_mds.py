"""Pins for the oracle's layout and classical MDS."""

import math

import numpy as np
import pytest

from oracle import layout, mds
from workloads import packed_distances, random_walk, walk_rng


def test_layout_matches_triu_order_and_roundtrips():
    iu, ju = np.triu_indices(64, 1)
    assert [layout.idx(int(i), int(j)) for i, j in zip(iu, ju)] == list(range(2016))
    x = np.random.default_rng(0).uniform(0, 5, 2016)
    d = layout.unpack(x)
    assert np.array_equal(d, d.T) and np.all(np.diag(d) == 0)
    assert np.array_equal(layout.pack(d), x)


def test_jacobi_matches_lapack():
    rng = np.random.default_rng(1)
    for n in (2, 5, 16, 64):
        a = rng.standard_normal((n, n))
        a = a + a.T
        ev, vec = mds.jacobi_eigh(a)
        ref = np.linalg.eigvalsh(a)
        assert np.allclose(np.sort(ev), ref, rtol=0, atol=1e-10 * np.abs(ref).max())
        assert np.allclose(vec.T @ vec, np.eye(n), atol=1e-12)
        assert np.allclose(a @ vec, vec * ev[None, :], atol=1e-10 * np.abs(ref).max())


def _collinear(n=64):
    return np.stack([np.arange(n, dtype=np.float64), np.zeros(n), np.zeros(n)], axis=1)


@pytest.mark.parametrize("solver", ["eigh", "jacobi"])
def test_collinear_chain_closed_form(solver):
    # D_ij = |i - j|: the Gram matrix of centred positions has one eigenvalue n(n^2 - 1) / 12
    x, lam = mds.classical_mds(packed_distances(_collinear()), solver=solver)
    assert lam[0] == pytest.approx(64 * (64 ** 2 - 1) / 12, rel=1e-12) == 21840
    assert abs(lam[1]) < 1e-9 and abs(lam[2]) < 1e-9
    assert np.allclose(mds.coords_distances(x), packed_distances(_collinear()), atol=1e-9)


@pytest.mark.parametrize("solver", ["eigh", "jacobi"])
def test_regular_polygon_closed_form(solver):
    n, rho = 64, 3.5
    ang = 2 * np.pi * np.arange(n) / n
    pts = np.stack([rho * np.cos(ang), rho * np.sin(ang), np.zeros(n)], axis=1)
    _, lam = mds.classical_mds(packed_distances(pts), solver=solver)
    assert lam[0] == pytest.approx(n * rho ** 2 / 2, rel=1e-12)
    assert lam[1] == pytest.approx(n * rho ** 2 / 2, rel=1e-12)
    assert abs(lam[2]) < 1e-9


def test_triangle_and_tetrahedron_by_hand():
    # equilateral triangle of side 1: centred Gram eigenvalues 1/2, 1/2, 0
    _, lam = mds.classical_mds(np.ones(3), n=3, solver="jacobi")
    assert np.allclose(lam, [0.5, 0.5, 0.0], atol=1e-14)
    # regular tetrahedron of side 1: 1/2, 1/2, 1/2
    _, lam = mds.classical_mds(np.ones(6), n=4, solver="jacobi")
    assert np.allclose(lam, [0.5, 0.5, 0.5], atol=1e-14)
    # right triangle with legs 3, 4: pairs (0,1)=3, (0,2)=4, (1,2)=5; trace of the Gram = sum d^2 / n
    x, lam = mds.classical_mds(np.array([3.0, 4.0, 5.0]), n=3, solver="jacobi")
    assert lam.sum() == pytest.approx((9 + 16 + 25) / 3, rel=1e-14)
    assert np.allclose(mds.coords_distances(x), [3, 4, 5], atol=1e-12)


@pytest.mark.parametrize("sigma", [None, 0.25])
def test_random_walk_recovered_exactly(sigma):
    for seed in range(3):
        coords = random_walk(64, walk_rng(99, seed), sigma)
        packed = packed_distances(coords)
        for solver in ("eigh", "jacobi"):
            x, lam = mds.classical_mds(packed, solver=solver)
            assert np.allclose(mds.coords_distances(x), packed, rtol=0, atol=1e-9)
            _, resid = mds.procrustes(x, coords)
            assert resid < 1e-9
            # centred Gram trace = sum of squared distances / n
            assert lam.sum() == pytest.approx(np.sum(packed ** 2) / 64, rel=1e-10)


def test_sign_convention_and_negative_clamp():
    coords = random_walk(64, walk_rng(5), None)
    x, _ = mds.classical_mds(packed_distances(coords))
    for k in range(3):
        assert x[np.argmax(np.abs(x[:, k])), k] > 0
    # a non-Euclidean map: a 4-point "square" whose diagonals are too long
    d = np.array([1.0, 3.0, 1.0, 1.0, 3.0, 1.0])
    x, lam = mds.classical_mds(d, n=4, solver="jacobi")
    ev = np.sort(np.linalg.eigvalsh(mds.double_centre(layout.unpack(d, 4))))[::-1][:3]
    assert np.allclose(lam, ev, atol=1e-12)
    for k in range(3):
        if lam[k] <= 0:
            assert np.all(x[:, k] == 0)


def test_procrustes_undoes_rotation_reflection_translation():
    rng = np.random.default_rng(8)
    y = rng.standard_normal((20, 3))
    q, _ = np.linalg.qr(rng.standard_normal((3, 3)))
    q[:, 0] *= -1
    x = y @ q + rng.standard_normal(3)
    aligned, resid = mds.procrustes(x, y)
    assert resid < 1e-12 and np.allclose(aligned, y, atol=1e-12)
    _, resid = mds.procrustes(x + rng.standard_normal(x.shape) * 0.1, y)
    assert resid > 0.01


def test_equivariance_under_scaling_and_bead_relabelling():
    """Distances scaled by c give coordinates scaled by c and eigenvalues by c^2; relabelling the
    beads relabels the coordinates (the sign convention follows the entries, not their index,
    wherever the largest magnitude is unique)."""
    rng = np.random.default_rng(3)
    for k in range(4):
        walk = random_walk(64, walk_rng(11, k), None)
        d = packed_distances(walk)
        x, lam = mds.classical_mds(d)
        xs, lams = mds.classical_mds(3.0 * d)
        assert np.allclose(xs, 3.0 * x, atol=1e-9 * np.abs(x).max())
        assert np.allclose(lams, 9.0 * lam, rtol=1e-12)
        perm = rng.permutation(64)
        xp, lamp = mds.classical_mds(packed_distances(walk[perm]))
        assert np.allclose(lamp, lam, rtol=1e-12)
        assert np.allclose(xp, x[perm], atol=1e-9 * np.abs(x).max())
