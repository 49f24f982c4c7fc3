"""Rigid stitching of adjacent tiles' point clouds — oracle, test infrastructure.

ParaChromo renders a chromosome-scale chain by recovering each tile's point
cloud and aligning adjacent tiles on their shared beads (section 5.5 and
Figure 4; the Kabsch residual after stitching is its coordinate-level
diagnostic).  Readings used here:

* tile k+1 is aligned onto the already-aligned tile k by the orthogonal map
  plus translation that best superposes its first O beads on tile k's last O
  beads (orthogonal Procrustes via the SVD, Schoenemann 1966 / Kabsch 1976).
  Reflections are allowed: a distance map fixes a point cloud only up to
  O(3), so adjacent tiles recovered independently can be mirror images;
* the residual of seam k is the RMS distance over the shared beads after the
  alignment;
* a bead shared by two tiles takes the mean of its two aligned positions.

The alternative reading, Kabsch's fit restricted to proper rotations
(det = +1, the determinant correction of the SVD solution), is available with
``proper=True``: where the best orthogonal map is a reflection, the sign of
the singular direction of the smallest singular value is flipped, which costs
4 sigma_3 in the sum of squared distances (the trace form of the objective).

Tile 0 keeps its own frame.  Shapes: tiles [L, 64, 3] -> chain
[(L-1)(64-O) + 64, 3] and residuals [L-1].
"""

from __future__ import annotations

import numpy as np


def align(x, y, proper: bool = False):
    """(R, shift): y ~ x @ R + shift, R orthogonal (3x3; a rotation with proper=True),
    minimising the squared error."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    xm, ym = x.mean(axis=0), y.mean(axis=0)
    u, _, vt = np.linalg.svd((x - xm).T @ (y - ym))
    r = u @ vt
    if proper and np.linalg.det(r) < 0:
        r = u @ np.diag([1.0, 1.0, -1.0]) @ vt
    return r, ym - xm @ r


def stitch_chain(tiles, overlap: int, proper: bool = False):
    tiles = np.asarray(tiles, dtype=np.float64)
    L, n, _ = tiles.shape
    stride = n - overlap
    chain = np.zeros(((L - 1) * stride + n, 3))
    count = np.zeros(chain.shape[0])
    resid = np.zeros(max(L - 1, 0))
    prev = tiles[0]
    chain[:n] += prev
    count[:n] += 1
    for k in range(1, L):
        x = tiles[k]
        r, shift = align(x[:overlap], prev[n - overlap:], proper)
        cur = x @ r + shift
        d = cur[:overlap] - prev[n - overlap:]
        resid[k - 1] = np.sqrt(np.mean(np.sum(d * d, axis=1)))
        chain[k * stride:k * stride + n] += cur
        count[k * stride:k * stride + n] += 1
        prev = cur
    return chain / count[:, None], resid
