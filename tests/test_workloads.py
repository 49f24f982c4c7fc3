"""The seeded input generators: shapes, determinism and seam-consistent chain windows."""

import numpy as np

from oracle import seam
from workloads import WORKLOADS, get, packed_distances, random_walk, reference_maps, walk_rng


def test_registry_shapes():
    assert [w.n_maps for w in WORKLOADS.values()] == [16, 2000, 16384, 32000, 531600]
    slab = get("genome_slab")
    assert slab.state_bytes() == 531600 * 2016 * 4
    assert get("chr22_chain").chain_beads == 1676


def test_walk_steps():
    c = random_walk(64, walk_rng(0, 1), None)
    steps = np.linalg.norm(np.diff(c, axis=0), axis=1)
    assert np.allclose(steps, 1.0) and np.all(c[0] == 0)
    c = random_walk(4000, walk_rng(0, 2), 0.25)
    logs = np.log(np.linalg.norm(np.diff(c, axis=0), axis=1))
    assert abs(logs.mean()) < 0.02 and abs(logs.std() - 0.25) < 0.02


def test_reference_maps_deterministic_fp32_and_subset():
    wl = get("genome_slab")
    a, b = reference_maps(wl, 1, regions=[0, 7, 2657])
    a2, _ = reference_maps(wl, 1, regions=[7])
    assert a.dtype == np.float32 and a.shape == (3, 2016)
    assert np.array_equal(a[1], a2[0])
    assert not np.array_equal(a, b)
    c = random_walk(64, walk_rng(1, wl.family, 7, 0), None)
    assert np.array_equal(a2[0], packed_distances(c).astype(np.float32))


def test_chain_windows_agree_on_every_seam():
    wl = get("chr22_chain")
    x0c, x0u = reference_maps(wl, 0)
    assert x0c.shape == (32, 2016)
    for ref in (x0c, x0u):
        d = seam.discrepancy_rms(ref[:, None, :].astype(np.float64), 12)
        assert np.all(d == 0.0)
    assert not np.array_equal(x0c, x0u)
