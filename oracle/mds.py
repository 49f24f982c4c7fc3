"""Classical (Torgerson) MDS — oracle, test infrastructure.

ChromoGen turns each final distance map into a 64-bead point cloud with a
distance-geometry initialiser (ParaChromo, section 3.1).  The initialiser here
is classical MDS:

    A = -1/2 (D o D),   B = J A J  with  J = I - 1 1^T / n,

the eigenpairs of B sorted by decreasing eigenvalue, the top three kept,
negative eigenvalues clamped to zero, and X = V_3 diag(sqrt(max(lambda, 0))).
For an exact Euclidean distance matrix B is the Gram matrix of the centred
coordinates, so X reproduces every distance.

Sign convention for each coordinate column: its entry of largest magnitude is
made positive (the lowest bead index wins a tie).

Eigen-solvers: ``numpy.linalg.eigh`` (LAPACK), or ``jacobi_eigh``, cyclic
Jacobi rotations run until the off-diagonal Frobenius norm is below
tol * ||A||_F (Golub & Van Loan, "Matrix Computations", cyclic Jacobi).
"""

from __future__ import annotations

import math

import numpy as np

from .layout import pair_table, unpack


def double_centre(d) -> np.ndarray:
    d = np.asarray(d, dtype=np.float64)
    n = d.shape[-1]
    j = np.eye(n) - np.full((n, n), 1.0 / n)
    return j @ (-0.5 * d * d) @ j


def jacobi_eigh(a, tol: float = 1e-13, max_sweeps: int = 100):
    """Eigenvalues (unsorted) and eigenvectors (columns) of a symmetric matrix."""
    a = np.array(a, dtype=np.float64, copy=True)
    n = a.shape[0]
    v = np.eye(n)
    scale = np.linalg.norm(a)
    if scale == 0.0:
        return np.zeros(n), v
    for _ in range(max_sweeps):
        off = math.sqrt(2.0 * float(np.sum(np.triu(a, 1) ** 2)))
        if off <= tol * scale:
            break
        for p in range(n - 1):
            for q in range(p + 1, n):
                apq = a[p, q]
                if apq == 0.0:
                    continue
                theta = (a[q, q] - a[p, p]) / (2.0 * apq)
                if abs(theta) > 1e150:  # theta^2 would overflow; t -> 1 / (2 theta)
                    t = 0.5 / theta
                else:
                    t = math.copysign(1.0, theta) / (abs(theta) + math.sqrt(theta * theta + 1.0))
                c = 1.0 / math.sqrt(t * t + 1.0)
                s = t * c
                # A <- R^T A R with R the rotation in the (p, q) plane.
                ap = a[:, p].copy()
                aq = a[:, q].copy()
                a[:, p] = c * ap - s * aq
                a[:, q] = s * ap + c * aq
                ap = a[p, :].copy()
                aq = a[q, :].copy()
                a[p, :] = c * ap - s * aq
                a[q, :] = s * ap + c * aq
                vp = v[:, p].copy()
                vq = v[:, q].copy()
                v[:, p] = c * vp - s * vq
                v[:, q] = s * vp + c * vq
    else:
        raise RuntimeError("Jacobi did not converge")
    return np.diag(a).copy(), v


def _top3(evals, evecs):
    order = np.argsort(-evals, kind="stable")[:3]
    lam = evals[order]
    vec = evecs[:, order]
    for k in range(vec.shape[1]):
        i = int(np.argmax(np.abs(vec[:, k])))
        if vec[i, k] < 0:
            vec[:, k] = -vec[:, k]
    return lam, vec


def classical_mds(packed, n: int = 64, solver: str = "eigh"):
    """(coords [n, 3], top-3 eigenvalues [3]) from one packed distance map."""
    b = double_centre(unpack(packed, n))
    if solver == "eigh":
        evals, evecs = np.linalg.eigh(b)
    elif solver == "jacobi":
        evals, evecs = jacobi_eigh(b)
    else:
        raise ValueError(solver)
    lam, vec = _top3(evals, evecs)
    coords = vec * np.sqrt(np.maximum(lam, 0.0))[None, :]
    return coords, lam


def coords_distances(coords) -> np.ndarray:
    """Packed pairwise distances [n(n-1)/2] of coordinates [n, d]."""
    x = np.asarray(coords, dtype=np.float64)
    rows, cols = pair_table(x.shape[0])
    diff = x[rows] - x[cols]
    return np.sqrt(np.sum(diff * diff, axis=1))


def procrustes(x, y):
    """Align x to y by translation and an orthogonal map (reflections allowed).

    Returns (aligned x, RMS residual).  Orthogonal Procrustes (Schoenemann, 1966):
    with centred x, y and U S V^T = svd(x^T y), the optimal map is U V^T.
    """
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    xc = x - x.mean(axis=0)
    yc = y - y.mean(axis=0)
    u, _, vt = np.linalg.svd(xc.T @ yc)
    aligned = xc @ (u @ vt) + y.mean(axis=0)
    return aligned, float(np.sqrt(np.mean(np.sum((aligned - y) ** 2, axis=1))))
