"""The C ABI on the host: the library loads, exports every symbol include/pc.h
declares, its host-side helpers agree with the oracle, and argument errors are
caught before any launch.  Nothing here touches a GPU."""

import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from tiled_genome_diffusion_amd import _lib
from oracle import philox, schedule, seam

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pc.h")


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^PC_API\s+[\w\s\*]*?\b(pc_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libpc.so is not built (python -m tiled_genome_diffusion_amd.build)")
    return _lib.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (pc_\w+)", out))
    assert set(names) <= exported
    assert set(names) == set(_lib.SIGNATURES)  # the binding declares exactly the header's entry points
    for n in names:
        assert getattr(lib, n) is not None


def test_version_and_status_strings(lib):
    assert "gfx950" in pc.pc_version()
    assert lib.pc_status_string(0) == b"ok"
    assert lib.pc_status_string(-4) == b"parameter out of range"


def test_schedule_matches_oracle_bitwise():
    for n in (50, 250, 500, 1000):
        a, b = pc.pc_ddim_schedule(n)
        want = schedule.ddim_pairs(n)
        assert np.array_equal(a, [p[0] for p in want])
        assert np.array_equal(b, [p[1] for p in want])
    with pytest.raises(pc.PCError):
        pc.pc_ddim_schedule(3)


def test_cosine_schedule_matches_oracle():
    ab = schedule.alpha_bar_from_betas(schedule.betas_cosine())
    for n in (50, 1000):
        a, b = pc.pc_ddim_schedule_cosine(n)
        want = schedule.ddim_pairs(n, ab=ab)
        assert np.allclose(a, [p[0] for p in want], rtol=1e-14, atol=0)
        assert np.allclose(b, [p[1] for p in want], rtol=1e-14, atol=0)
    with pytest.raises(pc.PCError):
        pc.pc_ddim_schedule_cosine(50, s=-0.1)


def test_seam_index_map_matches_oracle():
    for o in (2, 5, 12, 32):
        li, ri = seam.seam_pairs(o)
        got = pc.pc_seam_index_map(o)
        assert np.array_equal(got[:, 0], li) and np.array_equal(got[:, 1], ri)
    for bad in (1, 0, 33):
        with pytest.raises(pc.PCError):
            pc.pc_seam_index_map(bad)


def test_host_philox_matches_oracle():
    rng = np.random.default_rng(5)
    for _ in range(100):
        ctr = [int(v) for v in rng.integers(0, 2**32, 4, dtype=np.uint64)]
        seed = int(rng.integers(0, 2**63, dtype=np.uint64))
        assert pc.pc_philox_block(ctr, seed) == philox.block(ctr, philox.key_from_seed(seed))


def _lay(R=1, G=2, S=8, L=1, O=0):
    return _lib.Layout(R, G, S, L, O)


FAKE = ctypes.c_void_p(4096)   # never dereferenced: every call below fails validation first
W = (ctypes.c_float * 2)(0.0, 1.0)


@pytest.mark.parametrize("args,status", [
    (dict(state=None), -1),
    (dict(layout=_lay(R=0)), -2),
    (dict(layout=_lay(G=17)), -2),
    (dict(layout=_lay(R=32, L=5)), -2),
    (dict(layout=_lay(R=32, L=32, O=1)), -2),
    (dict(layout=_lay(R=32, L=32, O=33)), -2),
    (dict(layout=_lay(R=2**20, G=16, S=2**12)), -2),
    (dict(state=ctypes.c_void_p(4100)), -3),
    (dict(abar_t=0.0), -4),
    (dict(abar_t=1.0), -4),
    (dict(abar_next=1.5), -4),
    (dict(abar_t=0.5, abar_next=0.4), -4),
    (dict(eta=-1.0), -4),
    (dict(eta=float("nan")), -4),
    (dict(eta=5.0), -4),
    (dict(project=1), -4),
    (dict(pre_disc=FAKE), -4),
])
def test_step_validation(lib, args, status):
    a = dict(state=FAKE, layout=_lay(), abar_t=0.3, abar_next=0.5, eta=1.0, project=0, pre_disc=None)
    a.update(args)
    lay = a["layout"]
    st = lib.pc_ddim_cfg_step(a["state"], FAKE, FAKE, W, ctypes.byref(lay), a["abar_t"], a["abar_next"], a["eta"],
                              0, 1, a["project"], a["pre_disc"], None)
    assert st == status
    assert lib.pc_last_error() != b""


def test_other_validation(lib):
    lay = _lay()
    assert lib.pc_ddim_cfg_step_eps(FAKE, None, FAKE, W, ctypes.byref(lay), 0.3, 0.5, 1.0, 0, 1, 0, None, None) == -1
    assert lib.pc_ddim_cfg_step_eps(FAKE, FAKE, ctypes.c_void_p(4104), W, ctypes.byref(lay), 0.3, 0.5, 1.0, 0, 1, 0,
                                    None, None) == -3
    assert lib.pc_ddim_cfg_step_eps(FAKE, FAKE, FAKE, W, ctypes.byref(lay), 0.6, 0.5, 1.0, 0, 1, 0, None, None) == -4
    assert lib.pc_seam_project(FAKE, ctypes.byref(lay), None) == -2          # no chains
    assert lib.pc_seam_discrepancy(FAKE, ctypes.byref(lay), FAKE, None, None) == -2
    assert lib.pc_mds_recover(FAKE, -1, FAKE, None, 0, None) == -2
    assert lib.pc_mds_recover(FAKE, 10, FAKE, None, 999, None) == -4
    assert lib.pc_mds_recover(None, 10, FAKE, None, 0, None) == -1
    assert lib.pc_mds_recover(None, 0, None, None, 0, None) == 0          # empty batch: a no-op
    assert lib.pc_mds_recover(ctypes.c_void_p(4104), 10, FAKE, None, 0, None) == -3
    assert lib.pc_init_state(None, ctypes.byref(lay), 0, None) == -1
    assert lib.pc_kabsch_stitch(FAKE, ctypes.byref(lay), FAKE, FAKE, None) == -2            # no chains
    long_chain = _lay(R=2048, G=1, S=1, L=2048, O=12)
    assert lib.pc_kabsch_stitch(FAKE, ctypes.byref(long_chain), FAKE, FAKE, None) == -2     # chain_len > 1024
    short_seam = _lay(R=4, G=1, S=1, L=4, O=3)
    assert lib.pc_kabsch_stitch(FAKE, ctypes.byref(short_seam), FAKE, FAKE, None) == -2     # coplanar seams
    assert lib.pc_philox_fill(ctypes.c_void_p(4097), ctypes.byref(lay), 0, 0, None) == -3
    assert lib.pc_ddim_sample(FAKE, FAKE, FAKE, W, ctypes.byref(lay), 7, 1000, 1e-4, 0.02, 1.0, 0, 0, 1, None) == -4
    assert lib.pc_ddim_sample(FAKE, FAKE, FAKE, W, ctypes.byref(lay), 50, 1000, 1e-4, 0.02, 1.0, 0, 1, 1, None) == -4
    assert lib.pc_ddim_sample(FAKE, FAKE, FAKE, W, ctypes.byref(lay), 50, 1000, 1e-4, 0.02, 9.0, 0, 0, 1, None) == -4


def test_binding_rejects_host_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(16 * 2016)
    with pytest.raises(ValueError):
        pc.pc_init_state(x, pc.PCLayout(1, 2, 8), 0)


def test_mds_start_block_is_current_and_orthonormal(repo_root):
    """The committed start block of the MDS iteration is what its generator writes,
    orthonormal and orthogonal to the all-ones vector (the null vector of a doubly
    centred matrix) to float32 rounding."""
    import importlib.util

    csrc = os.path.join(repo_root, "tiled_genome_diffusion_amd", "csrc")
    spec = importlib.util.spec_from_file_location("mds_start", os.path.join(csrc, "mds_start.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    with open(os.path.join(csrc, "mds_start.hpp")) as f:
        text = f.read()
    got = np.array([float(v) for v in re.findall(r"(-?[0-9.]+e[-+][0-9]+)f", text)], dtype=np.float32)
    assert got.shape == (64 * 4,)
    q = got.reshape(64, 4).astype(np.float64)
    assert np.array_equal(got.reshape(64, 4), gen.start_block())
    assert np.abs(q.T @ q - np.eye(4)).max() < 1e-6
    assert np.abs(q.sum(axis=0)).max() < 1e-6
