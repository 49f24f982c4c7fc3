"""The whole reverse-diffusion loop, step by step — oracle, test infrastructure.

Layout of a batch: maps are indexed (r, g, s) for region (or tile) r, guidance
weight g and trajectory s, and the trajectory id that keys the noise is
t = (r G + g) S + s.

Independent regions: every map runs its own chain (ParaChromo, section 3.3:
no communication between tasks during denoising).

Chains: tiles k = 0 .. L-1 of one chain with the same (g, s) form one joint
tiled sample (ParaChromo, section 4.3.2).  Every tile takes its step, then
every K-th step the seams are projected (after the step, so a projection
also follows the last step when K divides the step count).

Initial state: x_T ~ N(0, 1) i.i.d. per packed entry (section 4.3.1: each
region starts from independent Gaussian noise), drawn from Philox slot 0.
"""

from __future__ import annotations

import numpy as np

from . import ddim, normals, philox, schedule, seam

P = 2016


def traj_id(r: int, g: int, s: int, G: int, S: int) -> int:
    return (r * G + g) * S + s


def noise(seed: int, slot: int, traj_ids) -> np.ndarray:
    """float64 [len(traj_ids), 2016] standard normals of one Philox step slot."""
    return normals.words_to_normals(philox.map_words(seed, traj_ids, slot, P))


def run_independent(x0c, x0u, w, traj_ids, seed: int, n_steps: int, eta: float,
                    record=(), T: int = 1000, beta_start: float = 1e-4, beta_end: float = 0.02):
    """Independent trajectories.  Row m of x0c/x0u/w/traj_ids describes map m.

    Returns (final states [M, P], {step: states}) where step counts completed
    DDIM steps (0 = x_T) for each step in ``record``.
    """
    x0c = np.asarray(x0c, dtype=np.float64)
    x0u = np.asarray(x0u, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64).reshape(-1, 1)
    traj_ids = np.asarray(traj_ids)
    x = noise(seed, 0, traj_ids)
    rec = {}
    if 0 in record:
        rec[0] = x.copy()
    for i, (a, a_next) in enumerate(schedule.ddim_pairs(n_steps, T, beta_start, beta_end)):
        z = noise(seed, i + 1, traj_ids) if eta != 0.0 else 0.0
        x = ddim.ddim_cfg_step(x, x0c, x0u, w, a, a_next, eta, z)
        if i + 1 in record:
            rec[i + 1] = x.copy()
    return x, rec


def run_chain(x0c_tiles, x0u_tiles, w, traj_ids, seed: int, n_steps: int, eta: float, overlap: int,
              project_every: int = 1, record=(), T: int = 1000, beta_start: float = 1e-4,
              beta_end: float = 0.02):
    """One chain of L tiles with B joint samples.

    x0c_tiles, x0u_tiles: [L, P]; w: [B]; traj_ids: [L, B].
    Returns (final [L, B, P], {step: states}, pre [n_steps, L-1, B], post [n_steps, L-1, B])
    where pre/post are the RMS seam discrepancies of each step before and after
    its projection (post equals pre on steps without a projection).
    """
    x0c = np.asarray(x0c_tiles, dtype=np.float64)[:, None, :]
    x0u = np.asarray(x0u_tiles, dtype=np.float64)[:, None, :]
    wv = np.asarray(w, dtype=np.float64).reshape(1, -1, 1)
    traj_ids = np.asarray(traj_ids)
    L, B = traj_ids.shape
    x = noise(seed, 0, traj_ids.reshape(-1)).reshape(L, B, P)
    rec = {}
    if 0 in record:
        rec[0] = x.copy()
    pre = np.zeros((n_steps, L - 1, B))
    post = np.zeros((n_steps, L - 1, B))
    for i, (a, a_next) in enumerate(schedule.ddim_pairs(n_steps, T, beta_start, beta_end)):
        z = noise(seed, i + 1, traj_ids.reshape(-1)).reshape(L, B, P) if eta != 0.0 else 0.0
        x = ddim.ddim_cfg_step(x, x0c, x0u, wv, a, a_next, eta, z)
        if L > 1:
            pre[i] = seam.discrepancy_rms(x, overlap)
            if (i + 1) % project_every == 0:
                x = seam.project(x, overlap)
            post[i] = seam.discrepancy_rms(x, overlap)
        if i + 1 in record:
            rec[i + 1] = x.copy()
    return x, rec, pre, post
