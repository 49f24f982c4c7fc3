"""ctypes declarations of libpc.so (include/pc.h).  Loading fails loudly if the
library has not been built; there is no fallback implementation."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpc.so")

c_float_p = ctypes.POINTER(ctypes.c_float)
c_double_p = ctypes.POINTER(ctypes.c_double)
c_u32_p = ctypes.POINTER(ctypes.c_uint32)
c_i32_p = ctypes.POINTER(ctypes.c_int32)
vp = ctypes.c_void_p


class Layout(ctypes.Structure):
    _fields_ = [("n_regions", ctypes.c_int32), ("n_guidance", ctypes.c_int32), ("n_traj", ctypes.c_int32),
                ("chain_len", ctypes.c_int32), ("overlap", ctypes.c_int32)]


# name -> (restype, argtypes), in the order of include/pc.h
SIGNATURES = {
    "pc_version": (ctypes.c_char_p, []),
    "pc_status_string": (ctypes.c_char_p, [ctypes.c_int32]),
    "pc_last_error": (ctypes.c_char_p, []),
    "pc_ddim_schedule": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                          c_double_p, c_double_p]),
    "pc_ddim_schedule_cosine": (ctypes.c_int32, [ctypes.c_int32, ctypes.c_int32, ctypes.c_double, ctypes.c_double,
                                                 c_double_p, c_double_p]),
    "pc_init_state": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), ctypes.c_uint64, vp]),
    "pc_ddim_cfg_step": (ctypes.c_int32, [vp, vp, vp, c_float_p, ctypes.POINTER(Layout), ctypes.c_double,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.c_int32, vp, vp]),
    "pc_ddim_cfg_step_eps": (ctypes.c_int32, [vp, vp, vp, c_float_p, ctypes.POINTER(Layout), ctypes.c_double,
                                              ctypes.c_double, ctypes.c_double, ctypes.c_uint64, ctypes.c_uint32,
                                              ctypes.c_int32, vp, vp]),
    "pc_ddim_sample": (ctypes.c_int32, [vp, vp, vp, c_float_p, ctypes.POINTER(Layout), ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                        ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32, vp]),
    "pc_seam_project": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), vp]),
    "pc_seam_discrepancy": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), vp, vp, vp]),
    "pc_seam_mean_abs": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), vp, vp]),
    "pc_mds_recover": (ctypes.c_int32, [vp, ctypes.c_int64, vp, vp, ctypes.c_int32, vp]),
    "pc_kabsch_stitch": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), vp, vp, vp]),
    "pc_kabsch_stitch_proper": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), vp, vp, vp]),
    "pc_set_max_dispatch_items": (ctypes.c_int32, [ctypes.c_uint64]),
    "pc_philox_block": (ctypes.c_int32, [c_u32_p, c_u32_p, ctypes.c_uint64]),
    "pc_philox_fill": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), ctypes.c_uint64, ctypes.c_uint32, vp]),
    "pc_normal_fill": (ctypes.c_int32, [vp, ctypes.POINTER(Layout), ctypes.c_uint64, ctypes.c_uint32, vp]),
    "pc_seam_index_map": (ctypes.c_int32, [c_i32_p, ctypes.c_int32]),
}

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run tiled_genome_diffusion_amd.build.build() "
                              "(hipcc --offload-arch=gfx950) first")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib
