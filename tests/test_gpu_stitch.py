"""GPU parity of chain stitching and of the paper-form seam discrepancy."""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import layout_of, map_index, run_steps, say, torch_dev, upload_refs
from oracle import seam, stitch
from workloads import Workload, get, random_walk, walk_rng

pytestmark = pytest.mark.gpu


def _orth(rng, reflect):
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if reflect:
        q[:, 0] *= -1
    return q


@pytest.mark.parametrize("L,O,n_chains,S", [(6, 12, 3, 4), (65, 4, 2, 3), (130, 12, 1, 2), (1024, 32, 1, 1)],
                         ids=["L6-O12", "L65-O4", "L130-O12", "L1024-O32"])
def test_stitch_synthetic_rigid_motions(L, O, n_chains, S):
    """Per-tile random rotations, reflections and shifts undone; chains longer than 64
    tiles cross the 64-tile chunks the fits are composed in, and 1024 is the longest
    chain the entry point accepts."""
    torch, dev = torch_dev()
    rng = np.random.default_rng(L * 100 + O)
    stride = 64 - O
    lay = pc.PCLayout(n_chains * L, 1, S, L, O)
    say(f"stitch: per-tile random rigid motions and reflections, L={L} O={O} chains={n_chains} S={S}")
    coords = np.zeros((n_chains * L, 1, S, 64, 3), dtype=np.float32)
    for c in range(n_chains):
        for s in range(S):
            walk = random_walk((L - 1) * stride + 64, walk_rng(c, s, 77), None)
            for k in range(L):
                t = walk[k * stride:k * stride + 64]
                coords[c * L + k, 0, s] = t @ _orth(rng, (k + s) % 2 == 1) + rng.standard_normal(3) * 5
    cd = torch.from_numpy(coords.reshape(-1)).to(dev)
    nb = (L - 1) * stride + 64
    chain = torch.empty(n_chains * S * nb * 3, dtype=torch.float32, device=dev)
    resid = torch.empty(n_chains * (L - 1) * S, dtype=torch.float32, device=dev)
    pc.pc_kabsch_stitch(cd, lay, chain, resid)
    got = chain.cpu().numpy().reshape(n_chains, S, nb, 3)
    res = resid.cpu().numpy().reshape(n_chains, L - 1, S)
    for c in range(n_chains):
        for s in range(S):
            want, wres = stitch.stitch_chain(coords[c * L:(c + 1) * L, 0, s].astype(np.float64), O)
            ext = np.abs(want).max()
            assert np.abs(got[c, s] - want).max() <= 1e-4 * ext
            # tiles were rounded to float32 after their motions: residuals sit at float32 rounding
            assert np.all(res[c, :, s] <= 1e-4 * ext) and np.all(wres <= 1e-5 * ext)


def _rot(rng):
    q = _orth(rng, False)
    if np.linalg.det(q) < 0:
        q[:, 0] *= -1
    return q


@pytest.mark.parametrize("mirror_every", [0, 3], ids=["rotations", "mirrored-tiles"])
def test_stitch_proper_matches_oracle(mirror_every):
    """Stitching restricted to rotations (det +1) against the oracle's Kabsch fit with the
    determinant correction.  Tiles moved by rotations only are stitched exactly; a mirrored
    tile cannot be superposed, and its seams keep a residual of the order of the shared
    block's size.  Residuals are compared everywhere; a mirrored seam's rotation is unique
    only when the two smallest singular values of its cross-covariance are apart, so chain
    coordinates are compared up to the first seam where they are not."""
    torch, dev = torch_dev()
    rng = np.random.default_rng(5 + mirror_every)
    L, O, S = 9, 12, 6
    stride = 64 - O
    lay = pc.PCLayout(L, 1, S, L, O)
    say(f"stitch, rotations only: L={L} O={O} S={S}, every {mirror_every or 'no'}th tile mirrored")
    coords = np.zeros((L, 1, S, 64, 3), dtype=np.float32)
    for s in range(S):
        walk = random_walk((L - 1) * stride + 64, walk_rng(s, 3, 91), None)
        for k in range(L):
            m = _rot(rng)
            if mirror_every and k % mirror_every == mirror_every - 1:
                m = m @ np.diag([1.0, 1.0, -1.0])
            coords[k, 0, s] = walk[k * stride:k * stride + 64] @ m + rng.standard_normal(3) * 5
    cd = torch.from_numpy(coords.reshape(-1)).to(dev)
    nb = (L - 1) * stride + 64
    chain = torch.empty(S * nb * 3, dtype=torch.float32, device=dev)
    resid = torch.empty((L - 1) * S, dtype=torch.float32, device=dev)
    pc.pc_kabsch_stitch_proper(cd, lay, chain, resid)
    got = chain.cpu().numpy().reshape(S, nb, 3)
    res = resid.cpu().numpy().reshape(L - 1, S)
    for s in range(S):
        tiles = coords[:, 0, s].astype(np.float64)
        want, wres = stitch.stitch_chain(tiles, O, proper=True)
        ext = np.abs(want).max()
        assert np.allclose(res[:, s], wres, atol=1e-4 * ext, rtol=1e-3)
        if not mirror_every:
            assert np.all(wres <= 1e-5 * ext) and np.abs(got[s] - want).max() <= 1e-4 * ext
            continue
        assert wres.max() > 0.05
        # compare the chain up to the first tile whose fit is not unique to float32 precision
        upto = L
        for k in range(1, L):
            x, y = tiles[k][:O], tiles[k - 1][stride:]
            sig = np.linalg.svd((x - x.mean(0)).T @ (y - y.mean(0)), compute_uv=False)
            if (sig[1] - sig[2]) < 0.05 * sig[0]:
                upto = k
                break
        n_ok = (upto - 1) * stride + 64 - (O if upto < L else 0)
        assert upto >= 2
        assert np.abs(got[s, :n_ok] - want[:n_ok]).max() <= 1e-4 * ext


def test_stitch_end_to_end_chr22():
    torch, dev = torch_dev()
    wl = get("chr22_chain")
    lay = layout_of(wl)
    say("stitch: chr22 chain sampled, MDS, stitched")
    refs = upload_refs(wl, 0)
    _, state, _ = run_steps(wl, 0, 50, [0], set(), refs=refs)
    coords = torch.empty(lay.n_maps * 192, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(state, coords)
    nb = wl.chain_beads
    chain = torch.empty(wl.n_guidance * wl.n_traj * nb * 3, dtype=torch.float32, device=dev)
    resid = torch.empty(lay.n_seams * wl.n_guidance * wl.n_traj, dtype=torch.float32, device=dev)
    pc.pc_kabsch_stitch(coords, lay, chain, resid)
    xyz = coords.cpu().numpy().reshape(lay.n_maps, 64, 3)
    got = chain.cpu().numpy().reshape(wl.n_guidance, wl.n_traj, nb, 3)
    res = resid.cpu().numpy().reshape(wl.chain_len - 1, wl.n_guidance, wl.n_traj)
    for g, s in [(0, 0), (1, 5), (0, 255)]:
        rows = [map_index(wl, k, g, s) for k in range(wl.chain_len)]
        want, wres = stitch.stitch_chain(xyz[rows].astype(np.float64), wl.overlap)
        ext = np.abs(want).max()
        assert np.abs(got[g, s] - want).max() <= 1e-4 * ext
        assert np.allclose(res[:, g, s], wres, atol=1e-4 * ext, rtol=1e-3)
        # the final maps are the reference windows of one chain walk: the seams close up
        assert wres.max() <= 1e-3


def test_seam_mean_abs_matches_oracle():
    torch, dev = torch_dev()
    wl = get("chr22_chain")
    lay = layout_of(wl)
    say("paper-form seam discrepancy on an unprojected and a projected chain state")
    refs = upload_refs(wl, 1)
    _, state, _ = run_steps(wl, 1, 50, [0], set(), project=False, refs=refs, stop_after=10)
    out = torch.empty(lay.n_seams * wl.n_guidance, dtype=torch.float32, device=dev)
    pc.pc_seam_mean_abs(state, lay, out)
    got = out.cpu().numpy().reshape(wl.chain_len - 1, wl.n_guidance)
    x = state.view(wl.chain_len, wl.n_guidance, wl.n_traj, 2016).cpu().numpy().astype(np.float64)
    for g in range(wl.n_guidance):
        want = seam.discrepancy_mean_abs(x[:, g], wl.overlap)
        assert np.allclose(got[:, g], want, rtol=1e-5, atol=1e-6)
        assert np.all(want > 0)
    pc.pc_seam_project(state, lay)
    pc.pc_seam_mean_abs(state, lay, out)
    assert torch.count_nonzero(out).item() == 0
