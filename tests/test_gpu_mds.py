"""GPU parity of batched classical MDS."""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import DIST_RTOL, layout_of, rel_dist_err, run_steps, say, torch_dev, upload_refs
from oracle import layout, mds
from workloads import get, packed_distances, pseudo_euclidean_map, random_walk, walk_rng

pytestmark = pytest.mark.gpu


def gpu_mds(maps_np, max_iters=0):
    torch, dev = torch_dev()
    maps = torch.from_numpy(np.ascontiguousarray(maps_np, dtype=np.float32)).to(dev)
    n = maps_np.shape[0]
    coords = torch.empty(n * 64 * 3, dtype=torch.float32, device=dev)
    eig = torch.empty(n * 3, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(maps, coords, eig, max_iters)
    return coords.cpu().numpy().reshape(n, 64, 3), eig.cpu().numpy().reshape(n, 3)


def dist_err(coords, maps_oracle_coords):
    """Per-map max |D_gpu - D_oracle| / max D_oracle, worst over maps."""
    worst = 0.0
    for c, o in zip(coords, maps_oracle_coords):
        worst = max(worst, rel_dist_err(mds.coords_distances(c), mds.coords_distances(o)))
    return worst


def test_exact_walk_maps():
    say("mds on exact walk maps")
    walks = [random_walk(64, walk_rng(7, k), None if k % 2 else 0.25) for k in range(64)]
    maps = np.array([packed_distances(w) for w in walks], dtype=np.float32)
    coords, eig = gpu_mds(maps)
    oc = [mds.classical_mds(m.astype(np.float64))[0] for m in maps]
    assert dist_err(coords, oc) <= DIST_RTOL
    for c, w in zip(coords, walks):
        _, resid = mds.procrustes(c.astype(np.float64), w)
        assert resid <= 1e-4 * np.abs(w - w.mean(axis=0)).max()
    for c in coords:   # sign convention
        for k in range(3):
            assert c[np.argmax(np.abs(c[:, k])), k] > 0


def test_closed_form_shapes():
    say("mds closed forms")
    line = np.stack([np.arange(64.0), np.zeros(64), np.zeros(64)], 1)
    ang = 2 * np.pi * np.arange(64) / 64
    ring = np.stack([3.5 * np.cos(ang), 3.5 * np.sin(ang), np.zeros(64)], 1)
    maps = np.array([packed_distances(line), packed_distances(ring), np.zeros(2016)], dtype=np.float32)
    coords, eig = gpu_mds(maps)
    assert eig[0, 0] == pytest.approx(21840.0, rel=1e-5)
    assert abs(eig[0, 1]) < 1e-2 and abs(eig[0, 2]) < 1e-2
    assert eig[1, 0] == pytest.approx(64 * 3.5 ** 2 / 2, rel=1e-5)
    assert eig[1, 1] == pytest.approx(64 * 3.5 ** 2 / 2, rel=1e-5)
    for k, pts in ((0, line), (1, ring)):
        assert rel_dist_err(mds.coords_distances(coords[k]), packed_distances(pts)) <= DIST_RTOL
    assert np.all(coords[2] == 0.0) and np.all(eig[2] == 0.0)   # all-zero map


def test_final_maps_of_the_sampler():
    wl = get("region_ensemble")
    say("mds on the 2000 final maps of region_ensemble")
    torch, dev = torch_dev()
    refs = upload_refs(wl, 2)
    _, state, _ = run_steps(wl, 2, 50, [0], set(), refs=refs)
    final = state.view(wl.n_maps, 2016).cpu().numpy()
    coords, _ = gpu_mds(final)
    oc = [mds.classical_mds(m.astype(np.float64))[0] for m in final]
    assert dist_err(coords, oc) <= DIST_RTOL


def test_non_euclidean_maps():
    # guided mixtures (w = 0.5) of two walk maps are not Euclidean: B has negative eigenvalues.
    # Noisy walk maps: relative noise 1e-3.
    say("mds on non-Euclidean maps")
    rng = np.random.default_rng(3)
    maps = []
    for k in range(48):
        a = packed_distances(random_walk(64, walk_rng(11, k, 0), None))
        b = packed_distances(random_walk(64, walk_rng(11, k, 1), None))
        maps.append(0.5 * (a + b) if k % 2 == 0 else a * (1 + 1e-3 * rng.standard_normal(2016)))
    maps = np.array(maps, dtype=np.float32)
    coords, eig = gpu_mds(maps, max_iters=256)
    oc, ol = zip(*[mds.classical_mds(m.astype(np.float64)) for m in maps])
    assert dist_err(coords, oc) <= DIST_RTOL
    assert np.allclose(eig, np.array(ol), rtol=1e-4, atol=1e-4 * np.abs(np.array(ol)).max())


def test_hidden_third_eigenvalue():
    # Maps whose Gram matrix has negative eigenvalues larger in magnitude than the
    # third wanted one: a block-4 iteration by magnitude misses lambda_3 and the
    # solver must deflate the negative directions and iterate again.
    say("mds on pseudo-Euclidean maps that hide lambda_3")
    folds = [(1.0, -1.0, 3.0, -4.0), (0.0, 2.0, -2.0, 5.0, -5.0), (1.0, -1.0)]
    maps = np.array([pseudo_euclidean_map(walk_rng(13, k), folds=folds[k % 3]) for k in range(36)])
    hidden = 0
    for m in maps:
        ev = np.linalg.eigvalsh(mds.double_centre(layout.unpack(m.astype(np.float32).astype(np.float64))))
        top4 = ev[np.argsort(-np.abs(ev))[:4]]
        hidden += not np.all(np.isin(np.sort(ev)[::-1][:3], top4))
    assert hidden >= 20
    coords, eig = gpu_mds(maps.astype(np.float32), max_iters=256)
    oc, ol = zip(*[mds.classical_mds(m.astype(np.float32).astype(np.float64)) for m in maps])
    assert dist_err(coords, oc) <= DIST_RTOL
    assert np.allclose(eig, np.array(ol), rtol=1e-4, atol=1e-4 * np.abs(np.array(ol)).max())


def test_hidden_third_eigenvalue_default_budget():
    # the same maps with the default iteration budget
    say("mds on pseudo-Euclidean maps, default budget")
    folds = [(1.0, -1.0, 3.0, -4.0), (0.0, 2.0, -2.0, 5.0, -5.0), (1.0, -1.0)]
    maps = np.array([pseudo_euclidean_map(walk_rng(13, k), folds=folds[k % 3]) for k in range(36)], dtype=np.float32)
    coords, _ = gpu_mds(maps)
    oc = [mds.classical_mds(m.astype(np.float64))[0] for m in maps]
    assert dist_err(coords, oc) <= DIST_RTOL


def test_empty_batch_is_a_no_op():
    torch, dev = torch_dev()
    say("mds on an empty batch")
    maps = torch.empty(0, dtype=torch.float32, device=dev)
    coords = torch.empty(0, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(maps, coords)
    torch.cuda.synchronize()


def test_noise_maps_stay_finite_and_ordered():
    # maps with no geometry at all (what a sampler fed random noise predictions ends on):
    # the iteration may hit its cap, but every output is finite, the eigenvalues come out in
    # descending order, and two runs agree bitwise
    say("mds on pure-noise maps")
    rng = np.random.default_rng(9)
    maps = np.abs(rng.standard_normal((256, 2016)) * 10).astype(np.float32)
    coords, eig = gpu_mds(maps)
    coords2, eig2 = gpu_mds(maps)
    assert np.all(np.isfinite(coords)) and np.all(np.isfinite(eig))
    assert np.all(eig[:, 0] >= eig[:, 1]) and np.all(eig[:, 1] >= eig[:, 2])
    assert np.array_equal(coords, coords2) and np.array_equal(eig, eig2)


def test_batch_slices_match_the_whole_batch():
    # one map, and batches that start inside a larger allocation (the maps are copied into
    # LDS by 16-byte lanes from any 16-byte aligned start): bitwise the rows of the whole run
    torch, dev = torch_dev()
    say("mds on slices of a batch")
    walks = [random_walk(64, walk_rng(21, k), 0.25) for k in range(13)]
    maps = torch.from_numpy(np.array([packed_distances(w) for w in walks], dtype=np.float32)).to(dev)
    n = maps.shape[0]
    whole = torch.empty(n * 64 * 3, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(maps, whole)
    whole = whole.view(n, 64, 3)
    for lo, hi in ((0, 1), (12, 13), (5, 6), (3, 10), (1, 13)):
        out = torch.empty((hi - lo) * 64 * 3, dtype=torch.float32, device=dev)
        pc.pc_mds_recover(maps[lo:hi], out)
        assert torch.equal(out.view(hi - lo, 64, 3), whole[lo:hi])


def test_scaling_the_distances_by_four_scales_the_output_exactly():
    """Every test and threshold of the kernel is relative, so distances times 4 (exact in
    float32) give coordinates times 4 and eigenvalues times 16, bit for bit: on exact walk
    maps, noisy ones and maps that are not Euclidean."""
    say("mds: scale equivariance")
    rng = np.random.default_rng(17)
    walks = [random_walk(64, walk_rng(19, k), None) for k in range(24)]
    exact = np.array([packed_distances(w) for w in walks], dtype=np.float32)
    noisy = (exact * (1.0 + 1e-3 * rng.standard_normal(exact.shape))).astype(np.float32)
    mixed = (0.5 * (exact + np.roll(exact, 1, axis=0))).astype(np.float32)
    maps = np.concatenate([exact, noisy, mixed])
    c1, e1 = gpu_mds(maps)
    c4, e4 = gpu_mds(maps * np.float32(4.0))
    assert np.array_equal(c4, c1 * np.float32(4.0))
    assert np.array_equal(e4, e1 * np.float32(16.0))
