"""Seeded 3D polymer random walks and their packed distance maps.

A region of the genome is 64 beads of 20 kb (ParaChromo, section 3.2); the
denoiser works on the region's pairwise distance map.  With no trained model
to sample from, the reference maps the stand-in denoiser pulls towards are the
distance maps of seeded random walks: bead 0 at the origin, each next bead one
step along an isotropic Gaussian direction, with either unit step length or a
length drawn from LogNormal(0, sigma).

Packed order: the strict upper triangle, row-major, i.e. the pairs (i, j) with
i < j in the order numpy's ``triu_indices(n, 1)`` lists them.
"""

from __future__ import annotations

import numpy as np


def walk_rng(*keys: int) -> np.random.Generator:
    """PCG64 generator seeded from a tuple of non-negative integers."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(keys))))


def random_walk(n_beads: int, rng: np.random.Generator, step_sigma: float | None = None) -> np.ndarray:
    """Coordinates [n_beads, 3] (float64) of a 3D random walk starting at the origin.

    Directions are normalised standard-normal 3-vectors.  Step lengths are 1, or
    exp(N(0, step_sigma^2)) when ``step_sigma`` is given.
    """
    if n_beads < 1:
        raise ValueError("n_beads must be >= 1")
    g = rng.standard_normal((n_beads - 1, 3))
    d = g / np.linalg.norm(g, axis=1, keepdims=True)
    if step_sigma is None:
        lengths = np.ones(n_beads - 1)
    else:
        lengths = rng.lognormal(mean=0.0, sigma=step_sigma, size=n_beads - 1)
    coords = np.zeros((n_beads, 3))
    coords[1:] = np.cumsum(d * lengths[:, None], axis=0)
    return coords


def packed_distances(coords: np.ndarray) -> np.ndarray:
    """Euclidean distances of all bead pairs i < j, row-major strict upper triangle (float64)."""
    n = coords.shape[0]
    iu, ju = np.triu_indices(n, 1)
    diff = coords[iu] - coords[ju]
    return np.sqrt(np.einsum("ij,ij->i", diff, diff))
