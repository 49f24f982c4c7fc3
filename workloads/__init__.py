"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This package holds only input generation: polymer random walks, their packed
distance maps, and the registry of workload shapes.  It contains none of the
sampler's arithmetic (no schedule, denoiser, guidance, DDIM update, seam
projection or MDS) and imports neither the oracle nor the HIP library, so both
sides can take their inputs from here without sharing any of the method.
"""

from .configs import (  # noqa: F401
    BEADS,
    BETA_END,
    BETA_START,
    PACKED,
    T_TRAIN,
    WORKLOADS,
    Workload,
    get,
    reference_maps,
    reference_walks,
)
from .walks import packed_distances, pseudo_euclidean_map, random_walk, walk_rng  # noqa: F401
