"""Registry of the synthetic workloads and their seeded reference maps.

Shapes follow the pages' workloads: 64-bead regions (ParaChromo, section 3.2),
two guidance settings per region, ensembles of stochastic samples, and the
chr22 tiling of 32 windows sharing 12 beads with each neighbour, 1676 beads in
all (ParaChromo, sections 3.2 and 5.5).  1676 = 31 * 52 + 64, so adjacent tiles
start 52 beads apart.

Every input is synthetic: reference maps are distance maps of seeded random
walks (see ``walks``), rounded to float32 once so both sides of a comparison
read identical bits.  Walk seeds are ``(base_seed, family, region, role)``
with role 0 for the conditional and 1 for the unconditional reference.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .walks import packed_distances, random_walk, walk_rng

BEADS = 64                      # beads per region / tile
PACKED = BEADS * (BEADS - 1) // 2   # 2016 packed distances per map
T_TRAIN = 1000                  # diffusion training steps of the schedule
BETA_START = 1e-4               # linear beta schedule endpoints
BETA_END = 0.02


@dataclass(frozen=True)
class Workload:
    name: str
    summary: str
    n_regions: int          # R: independent regions, or tiles of the chains
    n_guidance: int         # G
    n_traj: int             # S: trajectories per (region, guidance)
    chain_len: int          # tiles per chain; 1 = independent regions
    overlap: int            # beads shared by adjacent tiles (chains only)
    stride: int             # bead offset between adjacent tiles (chains only)
    n_steps: tuple          # DDIM step counts (one, or a sweep)
    eta: float              # DDIM eta (0 deterministic, 1 stochastic)
    w: tuple                # guidance weights, one per g
    step_sigma: float | None  # None: unit steps; else LogNormal(0, sigma) step lengths
    family: int             # walk-seed family (chains that share a walk share it)

    @property
    def n_maps(self) -> int:
        return self.n_regions * self.n_guidance * self.n_traj

    @property
    def n_chains(self) -> int:
        return self.n_regions // self.chain_len

    @property
    def chain_beads(self) -> int:
        return (self.chain_len - 1) * self.stride + BEADS

    def state_bytes(self) -> int:
        return self.n_maps * PACKED * 4


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_region", "1 region, 8 trajectories x 2 guidance weights, 50 DDIM steps, eta=0",
                 1, 2, 8, 1, 0, 0, (50,), 0.0, (0.0, 1.0), None, 1),
        Workload("region_ensemble", "1 region, 1000 trajectories x 2 guidance weights, 50 steps, eta=1, "
                 "LogNormal(0,0.25) walk steps",
                 1, 2, 1000, 1, 0, 0, (50,), 1.0, (0.0, 1.0), 0.25, 2),
        Workload("chr22_chain", "chr22-like chain: 32 tiles at stride 52 (12-bead overlap), 256 trajectories "
                 "x 2 guidance weights, 50 steps, eta=1, seam projection every step",
                 32, 2, 256, 32, 12, 52, (50,), 1.0, (0.0, 1.0), None, 3),
        Workload("chr22_sweep", "same 32-tile chain, 1000 trajectories, w=1, step sweep 50/250/500/1000, eta=1, "
                 "seam projection every step",
                 32, 1, 1000, 32, 12, 52, (50, 250, 500, 1000), 1.0, (1.0,), None, 3),
        Workload("genome_slab", "2658 independent regions x 2 guidance weights x 100 trajectories "
                 "(531,600 maps), 50 steps, eta=1",
                 2658, 2, 100, 1, 0, 0, (50,), 1.0, (0.0, 1.0), None, 5),
    ]
}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def reference_walks(wl: Workload, base_seed: int, regions=None):
    """Walk coordinates behind the reference maps.

    Independent regions: dict role -> list of [64, 3] arrays for ``regions``.
    Chains: dict role -> list of [chain_beads, 3] arrays, one per chain.
    """
    out = {0: [], 1: []}
    if wl.chain_len == 1:
        regs = range(wl.n_regions) if regions is None else regions
        for r in regs:
            for role in (0, 1):
                out[role].append(random_walk(BEADS, walk_rng(base_seed, wl.family, int(r), role), wl.step_sigma))
    else:
        for c in range(wl.n_chains):
            for role in (0, 1):
                out[role].append(random_walk(wl.chain_beads, walk_rng(base_seed, wl.family, c, role),
                                             wl.step_sigma))
    return out


def reference_maps(wl: Workload, base_seed: int, regions=None):
    """(x0_cond, x0_uncond): float32 [n, 2016] packed reference maps.

    ``regions`` selects a subset of independent regions (all by default); chains
    always return every tile, tile k of chain c at row c * chain_len + k, taken
    from beads k*stride .. k*stride+63 of that chain's walk.
    """
    walks = reference_walks(wl, base_seed, regions)
    maps = []
    for role in (0, 1):
        rows = []
        if wl.chain_len == 1:
            for coords in walks[role]:
                rows.append(packed_distances(coords))
        else:
            for coords in walks[role]:
                for k in range(wl.chain_len):
                    rows.append(packed_distances(coords[k * wl.stride:k * wl.stride + BEADS]))
        maps.append(np.ascontiguousarray(np.array(rows, dtype=np.float64).astype(np.float32)))
    return maps[0], maps[1]
