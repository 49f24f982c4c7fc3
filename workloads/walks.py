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


def pseudo_euclidean_map(rng: np.random.Generator, n_beads: int = 64, folds=(1.0, -1.0), fold_scale: float = 0.8,
                         spread=(0.6, 0.5)) -> np.ndarray:
    """A packed map that no 3D point set realises, with large negative directions.

    Beads sit along a noisy line (x, plus two small Gaussian coordinates); each
    entry of ``folds`` adds a coordinate fold_scale * |x - c| whose squared
    differences are subtracted instead of added (a pseudo-Euclidean space of
    signature (3, len(folds))).  Squared distances below zero are clamped.  The
    double-centred Gram matrix of such a map has, besides its three wanted
    positive eigenvalues, negative ones larger in magnitude than the second and
    third: the case where an eigen-solver that ranks by magnitude can miss a
    wanted eigenvalue.
    """
    x1 = np.linspace(-10.0, 10.0, n_beads) + rng.normal(0.0, 0.05, n_beads)
    pos = np.stack([x1, rng.normal(0.0, spread[0], n_beads), rng.normal(0.0, spread[1], n_beads)], 1)
    neg = np.stack([fold_scale * np.abs(x1 - c) for c in folds], 1)
    iu, ju = np.triu_indices(n_beads, 1)
    d2 = ((pos[iu] - pos[ju]) ** 2).sum(1) - ((neg[iu] - neg[ju]) ** 2).sum(1)
    return np.sqrt(np.maximum(d2, 0.0))
