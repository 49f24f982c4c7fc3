"""GPU parity of the tiled chain path: the step kernel with fused seam
projection and discrepancy, the standalone projection and discrepancy, and the
invariants the projection guarantees."""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import STATE_RTOL, layout_of, map_index, normwise_err, run_steps, say, torch_dev, upload_refs
from oracle import sampler, seam
from workloads import Workload, get

pytestmark = pytest.mark.gpu


def column_rows(wl, cols, chain=0):
    """Map indices [L * len(cols)] of the sampled (g, s) columns of one chain, tile-major."""
    L = wl.chain_len
    return np.array([map_index(wl, chain * L + k, g, s) for k in range(L) for (g, s) in cols])


def oracle_columns(wl, seed, x0c, x0u, cols, n_steps, record, project_every=1, chain=0):
    L = wl.chain_len
    tiles = slice(chain * L, chain * L + L)
    tids = np.array([[map_index(wl, chain * L + k, g, s) for (g, s) in cols] for k in range(L)])
    w = np.array([wl.w[g] for (g, _) in cols])
    return sampler.run_chain(x0c[tiles], x0u[tiles], w, tids, seed, n_steps, wl.eta, wl.overlap,
                             project_every=project_every, record=record)


def seam_rows(wl, cols, chain=0):
    """Flat indices into the [n_seams][G][S] discrepancy array for the sampled columns."""
    L, G, S = wl.chain_len, wl.n_guidance, wl.n_traj
    return np.array([(chain * (L - 1) + j) * G * S + g * S + s for j in range(L - 1) for (g, s) in cols])


@pytest.mark.parametrize("seed", [0, 2])
def test_chr22_chain_full_size_sampled_columns(seed):
    wl = get("chr22_chain")
    cols = [(0, 0), (1, 0), (0, 255), (1, 137)]
    say(f"chr22_chain 16,384 maps seed={seed}, columns {cols}")
    refs = upload_refs(wl, seed)
    idx = column_rows(wl, cols)
    record = set(range(51))
    rec, _, discs = run_steps(wl, seed, 50, idx, record, pre_disc=True, refs=refs)
    _, orec, pre, _ = oracle_columns(wl, seed, refs[0], refs[1], cols, 50, record)
    worst = 0.0
    for s in sorted(record):
        worst = max(worst, normwise_err(rec[s], orec[s].reshape(-1, 2016)))
    say(f"  worst normwise error {worst:.3e}")
    assert worst <= STATE_RTOL
    # pre-projection discrepancy of every step, seams x columns
    srows = seam_rows(wl, cols)
    L = wl.chain_len
    for s in range(1, 51):
        got = discs[s][srows].reshape(L - 1, len(cols))
        want = pre[s - 1]
        scale = max(1.0, float(np.abs(orec[s]).max()))
        assert np.all(np.abs(got - want) <= 2 * STATE_RTOL * scale + 1e-5 * want), f"step {s}"
    assert np.all(discs[50] == 0.0)   # last step: sigma = 0 and both copies agree exactly


def test_projection_invariants_full_size():
    torch, dev = torch_dev()
    wl = get("chr22_chain")
    lay = layout_of(wl)
    say("projection invariants on 16,384 maps")
    refs = upload_refs(wl, 1)
    # same keys, with and without projection on the final step
    _, base, _ = run_steps(wl, 1, 50, [0], set(), refs=refs, stop_after=49)
    a_t, a_n = pc.pc_ddim_schedule(50)
    noproj = base.clone()
    pc.pc_ddim_cfg_step(noproj, refs[2], refs[3], list(wl.w), lay, a_t[49], a_n[49], 1.0, 1, 50,
                        project_seams=False)
    # a mid-chain step, where sigma > 0 and the copies disagree before projection
    mid = base.clone()
    pc.pc_ddim_cfg_step(mid, refs[2], refs[3], list(wl.w), lay, a_t[10], a_n[10], 1.0, 1, 11,
                        project_seams=False)
    mid_proj = base.clone()
    pc.pc_ddim_cfg_step(mid_proj, refs[2], refs[3], list(wl.w), lay, a_t[10], a_n[10], 1.0, 1, 11,
                        project_seams=True)
    rms = torch.empty(lay.n_seams * lay.n_guidance * lay.n_traj, dtype=torch.float32, device=dev)
    summary = torch.empty(2, dtype=torch.float32, device=dev)
    pc.pc_seam_discrepancy(mid_proj, lay, rms, summary)
    assert torch.count_nonzero(rms).item() == 0 and summary.cpu().tolist() == [0.0, 0.0]
    # entries outside the seams are bitwise those of the unprojected step
    li, ri = seam.seam_pairs(wl.overlap)
    mask = np.ones((wl.chain_len, 2016), dtype=bool)
    mask[:-1, li] = False
    mask[1:, ri] = False
    tile_of_map = (np.arange(lay.n_maps) // (wl.n_guidance * wl.n_traj)) % wl.chain_len
    keep = torch.as_tensor(mask[tile_of_map], device=dev)
    a = mid.view(lay.n_maps, 2016)
    b = mid_proj.view(lay.n_maps, 2016)
    assert torch.equal(a[keep], b[keep])
    # fused projection == unfused step then standalone projection, bitwise
    alt = mid.clone()
    pc.pc_seam_project(alt, lay)
    assert torch.equal(alt, mid_proj)
    # idempotent
    again = mid_proj.clone()
    pc.pc_seam_project(again, lay)
    assert torch.equal(again, mid_proj)
    # standalone discrepancy of the unprojected state matches the oracle on sampled columns
    pc.pc_seam_discrepancy(mid, lay, rms, summary)
    cols = [(0, 3), (1, 200)]
    idx = column_rows(wl, cols)
    st = mid.view(lay.n_maps, 2016)[torch.as_tensor(idx, device=dev)].cpu().numpy()
    st = st.reshape(wl.chain_len, len(cols), 2016).astype(np.float64)
    want = seam.discrepancy_rms(st, wl.overlap)
    got = rms.cpu().numpy()[seam_rows(wl, cols)].reshape(wl.chain_len - 1, len(cols))
    assert np.allclose(got, want, rtol=1e-5, atol=1e-6)
    all_rms = rms.cpu().numpy().astype(np.float64)
    s = summary.cpu().numpy()
    assert s[0] == pytest.approx(all_rms.mean(), rel=1e-6) and s[1] == all_rms.max()
    del noproj


@pytest.mark.parametrize("n_steps", [50, 250, 500, 1000])
def test_chr22_sweep_sampled_columns(n_steps):
    wl = get("chr22_sweep")
    cols = [(0, 0), (0, 999)]
    say(f"chr22_sweep 32,000 maps, {n_steps} steps")
    refs = upload_refs(wl, 0)
    idx = column_rows(wl, cols)
    record = {1, 10, 25, n_steps // 2, n_steps}
    rec, _, _ = run_steps(wl, 0, n_steps, idx, record, refs=refs)
    fin, orec, _, post = oracle_columns(wl, 0, refs[0], refs[1], cols, n_steps, record)
    for s in sorted(record):
        assert normwise_err(rec[s], orec[s].reshape(-1, 2016)) <= STATE_RTOL, f"step {s}"
    # w = 1: the chain ends on the conditional references
    x0c = refs[0].astype(np.float64)
    assert normwise_err(rec[n_steps].reshape(wl.chain_len, len(cols), 2016),
                        np.repeat(x0c[:, None, :], len(cols), axis=1)) <= STATE_RTOL


@pytest.mark.parametrize("L,O,K", [(2, 12, 1), (5, 2, 1), (3, 32, 1), (7, 12, 3)])
def test_chain_edge_cases(L, O, K):
    torch, dev = torch_dev()
    # two chains of L tiles; tile stride 64 - O; ragged S; interval K through the whole-loop entry point
    wl = Workload("edge_chain", "", 2 * L, 2, 5, L, O, 64 - O, (50,), 1.0, (0.0, 1.0), None, 8)
    say(f"chain edge L={L} O={O} K={K}")
    refs = upload_refs(wl, 3)
    lay = layout_of(wl)
    state = torch.empty(lay.n_maps * 2016, dtype=torch.float32, device=dev)
    pc.pc_ddim_sample(state, refs[2], refs[3], list(wl.w), lay, 50, wl.eta, 3, project_every=K)
    cols = [(g, s) for g in range(2) for s in range(5)]
    for chain in range(2):
        idx = column_rows(wl, cols, chain)
        got = state.view(lay.n_maps, 2016)[torch.as_tensor(idx, device=dev)].cpu().numpy()
        fin, _, _, _ = oracle_columns(wl, 3, refs[0], refs[1], cols, 50, set(), project_every=K, chain=chain)
        assert normwise_err(got, fin.reshape(-1, 2016)) <= STATE_RTOL


def test_whole_loop_with_drawn_x_T_matches_step_loop():
    # pc_ddim_sample draws x_T inside its first (seam-projecting) step: bitwise the same as
    # pc_init_state followed by the step loop, without reading the state's prior contents
    torch, dev = torch_dev()
    wl = get("chr22_chain")
    say("chr22_chain: whole loop with x_T drawn in the first step vs step loop")
    refs = upload_refs(wl, 5)
    _, state, _ = run_steps(wl, 5, 50, [0], set(), refs=refs)
    lay = layout_of(wl)
    s2 = torch.full_like(state, float("nan"))
    pc.pc_ddim_sample(s2, refs[2], refs[3], list(wl.w), lay, 50, wl.eta, 5, project_every=1)
    torch.cuda.synchronize()
    assert torch.equal(state, s2)
