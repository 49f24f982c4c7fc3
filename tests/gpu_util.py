"""Helpers of the GPU parity tests: running the HIP path through the C ABI on
seeded inputs and comparing with the oracle."""

from __future__ import annotations

import os
import sys

import numpy as np

import tiled_genome_diffusion_amd as pc
from workloads import PACKED, Workload, reference_maps

STATE_RTOL = 1e-5     # max |x_gpu - x_oracle| <= STATE_RTOL * max(1, max |x_oracle|), per map
DIST_RTOL = 1e-4      # max |D_gpu - D_oracle| <= DIST_RTOL * max D_oracle, per map


def torch_dev():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a GPU")
    return torch, torch.device("cuda:0")


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def layout_of(wl: Workload) -> pc.PCLayout:
    return pc.PCLayout(wl.n_regions, wl.n_guidance, wl.n_traj, wl.chain_len, wl.overlap if wl.chain_len > 1 else 0)


def upload_refs(wl: Workload, seed: int):
    torch, dev = torch_dev()
    x0c, x0u = reference_maps(wl, seed)
    return x0c, x0u, torch.from_numpy(x0c).to(dev), torch.from_numpy(x0u).to(dev)


def map_index(wl: Workload, r: int, g: int, s: int) -> int:
    return (r * wl.n_guidance + g) * wl.n_traj + s


# Largest normwise state error seen by any parity check of the session (reported at the end),
# and the largest of each kind per test.
WORST = {"state": 0.0, "checks": 0, "dist": 0.0, "dist_checks": 0}
WORST_BY_TEST: dict = {}


def _note(kind: str, err: float) -> None:
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    key = (kind, test)
    WORST_BY_TEST[key] = max(WORST_BY_TEST.get(key, 0.0), err)


def normwise_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """Largest per-map max |gpu - ref| / max(1, max |ref|) over the leading axes."""
    g = np.asarray(gpu, dtype=np.float64).reshape(-1, PACKED)
    r = np.asarray(ref, dtype=np.float64).reshape(-1, PACKED)
    scale = np.maximum(1.0, np.abs(r).max(axis=1))
    err = float((np.abs(g - r).max(axis=1) / scale).max())
    WORST["state"] = max(WORST["state"], err)
    WORST["checks"] += 1
    _note("state", err)
    return err


def rel_dist_err(dist_gpu: np.ndarray, dist_ref: np.ndarray) -> float:
    """max |D_gpu - D_ref| / max D_ref for one map's pairwise distances."""
    err = float(np.abs(np.asarray(dist_gpu) - np.asarray(dist_ref)).max() / np.asarray(dist_ref).max())
    WORST["dist"] = max(WORST["dist"], err)
    WORST["dist_checks"] += 1
    _note("dist", err)
    return err


def run_steps(wl: Workload, seed: int, n_steps: int, sample_idx, record, project: bool = True, pre_disc=False,
              refs=None, stop_after: int | None = None):
    """Run the HIP sampler step by step (the first ``stop_after`` steps of an n_steps schedule, all by
    default); return ({step: state rows at sample_idx}, final state tensor, {step: pre-projection RMS})."""
    torch, dev = torch_dev()
    lay = layout_of(wl)
    if refs is None:
        refs = upload_refs(wl, seed)
    _, _, x0c_d, x0u_d = refs
    state = torch.empty(lay.n_maps * PACKED, dtype=torch.float32, device=dev)
    idx = torch.as_tensor(np.asarray(sample_idx, dtype=np.int64), device=dev)
    view = state.view(lay.n_maps, PACKED)
    pc.pc_init_state(state, lay, seed)
    rec = {}
    discs = {}
    if 0 in record:
        rec[0] = view.index_select(0, idx).cpu().numpy()
    a_t, a_n = pc.pc_ddim_schedule(n_steps)
    chains = wl.chain_len > 1
    disc_buf = torch.empty(lay.n_seams * lay.n_guidance * lay.n_traj, dtype=torch.float32, device=dev) \
        if (chains and pre_disc) else None
    for i in range(n_steps if stop_after is None else stop_after):
        pc.pc_ddim_cfg_step(state, x0c_d, x0u_d, list(wl.w), lay, a_t[i], a_n[i], wl.eta, seed, i + 1,
                            project_seams=chains and project, pre_disc=disc_buf)
        if i + 1 in record:
            rec[i + 1] = view.index_select(0, idx).cpu().numpy()
        if disc_buf is not None:
            discs[i + 1] = disc_buf.cpu().numpy()
    torch.cuda.synchronize()
    return rec, state, discs
