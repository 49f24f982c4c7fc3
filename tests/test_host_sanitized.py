"""The library's host layer under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Every source of libpc.so is compiled for the host alone (hipcc --offload-host-only: argument
checks, schedules, the seam index map, host Philox and the launchers with their dispatch
slicing) with both sanitizers, and linked with the HIP stand-ins of tests/host/hip_stub.cpp,
which record kernel launches instead of running them.  tests/host/api_check.cpp then drives
every entry point: validation branches, launch geometry and slicing up to the largest layout
the boundary accepts, error propagation and the host helpers.  Any sanitizer report or failed
check fails the test.  No GPU is used."""

from __future__ import annotations

import hashlib
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from tiled_genome_diffusion_amd import build as libbuild

HOST = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host")
SAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
SAN_LINK = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _clangxx() -> str:
    path = os.path.join(os.path.dirname(os.path.realpath(libbuild.hipcc())), "..", "llvm", "bin", "clang++")
    if not os.path.exists(path):
        path = "/opt/rocm/llvm/bin/clang++"
    return path


def _run(cmd, cwd):
    res = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    if res.returncode != 0:
        raise AssertionError(f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return res


@pytest.fixture(scope="module")
def host_check_exe():
    srcs = [os.path.join(libbuild.CSRC, s) for s in libbuild.SOURCES]
    extra = [os.path.join(HOST, f) for f in ("hip_stub.cpp", "hip_stub.hpp", "api_check.cpp")]
    headers = [os.path.join(libbuild.CSRC, f) for f in sorted(os.listdir(libbuild.CSRC)) if f.endswith(".hpp")]
    h = hashlib.sha256()
    for p in srcs + extra + headers + [os.path.join(libbuild.ROOT, "include", "pc.h")]:
        with open(p, "rb") as f:
            h.update(f.read())
    out = os.path.join(tempfile.gettempdir(), f"pc_host_check_{h.hexdigest()[:16]}")
    exe = os.path.join(out, "api_check")
    if os.path.exists(exe):
        return exe
    work = out + ".tmp"
    shutil.rmtree(work, ignore_errors=True)
    os.makedirs(work)
    inc = ["-I", os.path.join(libbuild.ROOT, "include"), "-I", libbuild.CSRC, "-I", HOST]
    common = ["-O1", "-g", "-std=c++17", "-ffp-contract=off"]
    objs = []
    for s in srcs + [os.path.join(HOST, "hip_stub.cpp")]:
        o = os.path.join(work, os.path.basename(s) + ".o")
        _run([libbuild.hipcc(), "-x", "hip", "--offload-host-only", *common, *SAN_HOST, *inc, "-c", s, "-o", o], work)
        objs.append(o)
    o = os.path.join(work, "api_check.o")
    _run([_clangxx(), *common, *SAN_LINK, *inc, "-I", "/opt/rocm/include", "-D__HIP_PLATFORM_AMD__", "-c",
          os.path.join(HOST, "api_check.cpp"), "-o", o], work)
    objs.append(o)
    # the host halves refer to the device code objects by per-file symbols; nothing reads them here
    syms = set()
    for obj in objs:
        nm = _run(["nm", "-u", obj], work).stdout
        syms.update(re.findall(r"\b(__hip_fatbin_\w+)", nm))
    stub_c = os.path.join(work, "fatbin_stub.c")
    with open(stub_c, "w") as f:
        for s in sorted(syms):
            f.write(f"const char {s}[16] = {{0}};\n")
    o = os.path.join(work, "fatbin_stub.o")
    _run([_clangxx(), "-x", "c", "-c", stub_c, "-o", o], work)
    objs.append(o)
    _run([_clangxx(), *SAN_LINK, "-o", os.path.join(work, "api_check"), *objs], work)
    shutil.rmtree(out, ignore_errors=True)
    os.replace(work, out)
    return exe


def test_host_layer_clean_under_asan_and_ubsan(host_check_exe):
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([host_check_exe], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host checks passed" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
