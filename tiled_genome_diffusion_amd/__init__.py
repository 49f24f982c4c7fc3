"""Python binding of the gfx950 hot path of tiled, ensemble 3D-genome diffusion.

Every function has the name of the C entry point it wraps (include/pc.h) and
only marshals arguments: torch tensors supply device memory, torch's current
stream supplies the HIP stream, and all arithmetic runs in the HIP kernels of
libpc.so.  A negative status raises ``PCError``.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import numpy as np

from . import _lib

__all__ = ["PCError", "PCLayout", "PACKED", "BEADS", "pc_version", "pc_last_error", "pc_ddim_schedule",
           "pc_ddim_schedule_cosine", "pc_init_state", "pc_ddim_cfg_step", "pc_ddim_cfg_step_eps", "pc_ddim_sample", "pc_seam_project", "pc_seam_discrepancy",
           "pc_seam_mean_abs", "pc_mds_recover", "pc_kabsch_stitch", "pc_kabsch_stitch_proper", "pc_set_max_dispatch_items", "pc_philox_block", "pc_philox_fill", "pc_normal_fill", "pc_seam_index_map"]

BEADS = 64
PACKED = 2016


class PCError(RuntimeError):
    def __init__(self, status: int, func: str):
        lib = _lib.load()
        self.status = status
        super().__init__(f"{func}: {lib.pc_status_string(status).decode()} ({status}): "
                         f"{lib.pc_last_error().decode()}")


@dataclass(frozen=True)
class PCLayout:
    n_regions: int
    n_guidance: int
    n_traj: int
    chain_len: int = 1
    overlap: int = 0

    @property
    def n_maps(self) -> int:
        return self.n_regions * self.n_guidance * self.n_traj

    @property
    def n_seams(self) -> int:
        return (self.n_regions // self.chain_len) * (self.chain_len - 1) if self.chain_len > 1 else 0

    def c(self) -> _lib.Layout:
        return _lib.Layout(self.n_regions, self.n_guidance, self.n_traj, self.chain_len, self.overlap)


def _check(status: int, func: str) -> None:
    if status != 0:
        raise PCError(status, func)


def _dev(t, dtype, numel: int | None, name: str):
    """Device pointer of a contiguous torch tensor of the given dtype (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(t) -> ctypes.c_void_p:
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _torch():
    import torch

    return torch


def pc_version() -> str:
    return _lib.load().pc_version().decode()


def pc_last_error() -> str:
    return _lib.load().pc_last_error().decode()


def pc_ddim_schedule(n_steps: int, T: int = 1000, beta_start: float = 1e-4, beta_end: float = 0.02):
    """(abar_t, abar_next): float64 numpy arrays [n_steps]."""
    a = np.zeros(n_steps, dtype=np.float64)
    b = np.zeros(n_steps, dtype=np.float64)
    st = _lib.load().pc_ddim_schedule(n_steps, T, beta_start, beta_end, a.ctypes.data_as(_lib.c_double_p),
                                      b.ctypes.data_as(_lib.c_double_p))
    _check(st, "pc_ddim_schedule")
    return a, b


def pc_ddim_schedule_cosine(n_steps: int, T: int = 1000, s: float = 0.008, beta_max: float = 0.999):
    """(abar_t, abar_next) of the cosine schedule: float64 numpy arrays [n_steps]."""
    a = np.zeros(n_steps, dtype=np.float64)
    b = np.zeros(n_steps, dtype=np.float64)
    st = _lib.load().pc_ddim_schedule_cosine(n_steps, T, s, beta_max, a.ctypes.data_as(_lib.c_double_p),
                                             b.ctypes.data_as(_lib.c_double_p))
    _check(st, "pc_ddim_schedule_cosine")
    return a, b


def pc_init_state(state, layout: PCLayout, seed: int) -> None:
    t = _torch()
    lay = layout.c()
    _check(_lib.load().pc_init_state(_dev(state, t.float32, layout.n_maps * PACKED, "state"), ctypes.byref(lay),
                                     seed, _stream(state)), "pc_init_state")


def _weights(w, G: int):
    if len(w) != G:
        raise ValueError(f"need {G} guidance weights, got {len(w)}")
    return (ctypes.c_float * G)(*[float(v) for v in w])


def pc_ddim_cfg_step(state, x0_cond, x0_uncond, w, layout: PCLayout, abar_t: float, abar_next: float, eta: float,
                     seed: int, slot: int, project_seams: bool = False, pre_disc=None) -> None:
    t = _torch()
    lay = layout.c()
    n_ref = layout.n_regions * PACKED
    _check(_lib.load().pc_ddim_cfg_step(
        _dev(state, t.float32, layout.n_maps * PACKED, "state"), _dev(x0_cond, t.float32, n_ref, "x0_cond"),
        _dev(x0_uncond, t.float32, n_ref, "x0_uncond"), _weights(w, layout.n_guidance), ctypes.byref(lay),
        float(abar_t), float(abar_next), float(eta), seed, slot, int(bool(project_seams)),
        _dev(pre_disc, t.float32, layout.n_seams * layout.n_guidance * layout.n_traj, "pre_disc"),
        _stream(state)), "pc_ddim_cfg_step")


def pc_ddim_cfg_step_eps(state, eps_cond, eps_uncond, w, layout: PCLayout, abar_t: float, abar_next: float,
                         eta: float, seed: int, slot: int, project_seams: bool = False, pre_disc=None) -> None:
    t = _torch()
    lay = layout.c()
    n = layout.n_maps * PACKED
    _check(_lib.load().pc_ddim_cfg_step_eps(
        _dev(state, t.float32, n, "state"), _dev(eps_cond, t.float32, n, "eps_cond"),
        _dev(eps_uncond, t.float32, n, "eps_uncond"), _weights(w, layout.n_guidance), ctypes.byref(lay),
        float(abar_t), float(abar_next), float(eta), seed, slot, int(bool(project_seams)),
        _dev(pre_disc, t.float32, layout.n_seams * layout.n_guidance * layout.n_traj, "pre_disc"),
        _stream(state)), "pc_ddim_cfg_step_eps")


def pc_ddim_sample(state, x0_cond, x0_uncond, w, layout: PCLayout, n_steps: int, eta: float, seed: int,
                   project_every: int = 0, init: bool = True, T: int = 1000, beta_start: float = 1e-4,
                   beta_end: float = 0.02) -> None:
    t = _torch()
    lay = layout.c()
    n_ref = layout.n_regions * PACKED
    _check(_lib.load().pc_ddim_sample(
        _dev(state, t.float32, layout.n_maps * PACKED, "state"), _dev(x0_cond, t.float32, n_ref, "x0_cond"),
        _dev(x0_uncond, t.float32, n_ref, "x0_uncond"), _weights(w, layout.n_guidance), ctypes.byref(lay),
        n_steps, T, beta_start, beta_end, float(eta), seed, project_every, int(bool(init)), _stream(state)),
        "pc_ddim_sample")


def pc_seam_project(state, layout: PCLayout) -> None:
    t = _torch()
    lay = layout.c()
    _check(_lib.load().pc_seam_project(_dev(state, t.float32, layout.n_maps * PACKED, "state"), ctypes.byref(lay),
                                       _stream(state)), "pc_seam_project")


def pc_seam_discrepancy(state, layout: PCLayout, rms, summary=None) -> None:
    t = _torch()
    lay = layout.c()
    _check(_lib.load().pc_seam_discrepancy(
        _dev(state, t.float32, layout.n_maps * PACKED, "state"), ctypes.byref(lay),
        _dev(rms, t.float32, layout.n_seams * layout.n_guidance * layout.n_traj, "rms"),
        _dev(summary, t.float32, 2, "summary"), _stream(state)), "pc_seam_discrepancy")


def pc_seam_mean_abs(state, layout: PCLayout, out) -> None:
    t = _torch()
    lay = layout.c()
    _check(_lib.load().pc_seam_mean_abs(
        _dev(state, t.float32, layout.n_maps * PACKED, "state"), ctypes.byref(lay),
        _dev(out, t.float32, layout.n_seams * layout.n_guidance, "out"), _stream(state)), "pc_seam_mean_abs")


def pc_mds_recover(maps, coords, eigvals=None, max_iters: int = 0) -> None:
    t = _torch()
    n = maps.numel() // PACKED
    if maps.numel() != n * PACKED:
        raise ValueError("maps must hold whole 2016-value maps")
    _check(_lib.load().pc_mds_recover(_dev(maps, t.float32, None, "maps"), n,
                                      _dev(coords, t.float32, n * BEADS * 3, "coords"),
                                      _dev(eigvals, t.float32, n * 3, "eigvals"), max_iters, _stream(maps)),
           "pc_mds_recover")


def _stitch(name: str, coords, layout: PCLayout, chain, residual) -> None:
    t = _torch()
    lay = layout.c()
    n_chains = layout.n_regions // layout.chain_len
    n_beads = (layout.chain_len - 1) * (BEADS - layout.overlap) + BEADS
    _check(getattr(_lib.load(), name)(
        _dev(coords, t.float32, layout.n_maps * BEADS * 3, "coords"), ctypes.byref(lay),
        _dev(chain, t.float32, n_chains * layout.n_guidance * layout.n_traj * n_beads * 3, "chain"),
        _dev(residual, t.float32, layout.n_seams * layout.n_guidance * layout.n_traj, "residual"),
        _stream(coords)), name)


def pc_kabsch_stitch(coords, layout: PCLayout, chain, residual) -> None:
    _stitch("pc_kabsch_stitch", coords, layout, chain, residual)


def pc_kabsch_stitch_proper(coords, layout: PCLayout, chain, residual) -> None:
    """pc_kabsch_stitch with every fit restricted to rotations (det +1)."""
    _stitch("pc_kabsch_stitch_proper", coords, layout, chain, residual)


def pc_set_max_dispatch_items(items: int) -> None:
    """Cap the work-items of one kernel dispatch (0 restores the hardware limit); a diagnostic."""
    _check(_lib.load().pc_set_max_dispatch_items(int(items)), "pc_set_max_dispatch_items")


def pc_philox_block(ctr, seed: int):
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    out = (ctypes.c_uint32 * 4)()
    _check(_lib.load().pc_philox_block(out, c, seed), "pc_philox_block")
    return tuple(int(v) for v in out)


def pc_philox_fill(out, layout: PCLayout, seed: int, slot: int) -> None:
    t = _torch()
    lay = layout.c()
    _check(_lib.load().pc_philox_fill(_dev(out, t.int32, layout.n_maps * PACKED, "out"), ctypes.byref(lay), seed,
                                      slot, _stream(out)), "pc_philox_fill")


def pc_normal_fill(out, layout: PCLayout, seed: int, slot: int) -> None:
    t = _torch()
    lay = layout.c()
    _check(_lib.load().pc_normal_fill(_dev(out, t.float32, layout.n_maps * PACKED, "out"), ctypes.byref(lay), seed,
                                      slot, _stream(out)), "pc_normal_fill")


def pc_seam_index_map(overlap: int) -> np.ndarray:
    n = overlap * (overlap - 1) // 2
    out = np.zeros((max(n, 1), 2), dtype=np.int32)
    _check(_lib.load().pc_seam_index_map(out.ctypes.data_as(_lib.c_i32_p), overlap), "pc_seam_index_map")
    return out[:n]
