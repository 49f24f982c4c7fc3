"""Compile the HIP libraries for gfx950, in-tree.

libpc.so holds every kernel and the C ABI of include/pc.h.  libpc_ceiling.so
holds the bandwidth probes bench.py measures the HBM ceiling with (the step
kernel's access pattern without its arithmetic); it is not part of the C ABI.
All HIP code is built with packed-FP32 instructions disabled and without
implicit FMA contraction (kernels spell out their fused multiply-adds, so every
kernel that computes a value rounds it the same way).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpc.so")
SOURCES = ["api.hip", "step.hip", "chain.hip", "seam.hip", "mds.hip", "stitch.hip"]
CEILING_LIB = os.path.join(HERE, "libpc_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def command(out: str = LIB, sources=None) -> list[str]:
    return [hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared", "-fvisibility=hidden",
            "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unknown-pragmas",
            "-I", os.path.join(ROOT, "include"),
            "-o", out] + [os.path.join(CSRC, s) for s in (SOURCES if sources is None else sources)]


def _compile(lib: str, sources, verbose: bool) -> None:
    tmp = lib + ".tmp"
    cmd = command(tmp, sources)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode}): {' '.join(cmd)}")
    if verbose:
        sys.stderr.write(res.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile libpc.so and libpc_ceiling.so (always, even if present); return libpc.so's path."""
    _compile(LIB, SOURCES, verbose)
    _compile(CEILING_LIB, CEILING_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
