"""GPU parity of the step variant that takes the network's noise predictions
from buffers, and of the cosine schedule (a stride-1 eta = 1 run is the DDPM
ancestral sampler)."""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import STATE_RTOL, layout_of, map_index, normwise_err, say, torch_dev, upload_refs
from oracle import ddim, sampler, schedule, seam
from workloads import Workload, get

pytestmark = pytest.mark.gpu


def _eps_inputs(n, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((n, 2016)).astype(np.float32), rng.standard_normal((n, 2016)).astype(np.float32))


@pytest.mark.parametrize("eta", [0.0, 1.0])
def test_eps_step_independent(eta):
    torch, dev = torch_dev()
    wl = Workload("eps", "", 3, 2, 11, 1, 0, 0, (50,), eta, (0.0, 1.5), None, 7)
    lay = layout_of(wl)
    say(f"eps step, independent, eta={eta}")
    ec, eu = _eps_inputs(lay.n_maps, 1)
    ec_d, eu_d = torch.from_numpy(ec).to(dev), torch.from_numpy(eu).to(dev)
    state = torch.empty(lay.n_maps * 2016, dtype=torch.float32, device=dev)
    pc.pc_init_state(state, lay, 5)
    x = state.view(lay.n_maps, 2016).cpu().numpy().astype(np.float64)
    a_t, a_n = pc.pc_ddim_schedule(50)
    idx = np.arange(lay.n_maps)
    w = np.asarray(wl.w)[(idx // wl.n_traj) % wl.n_guidance][:, None]
    for i in (0, 1, 2, 30, 49):   # any (a, a') pair: the buffers stand for one network call each
        pc.pc_ddim_cfg_step_eps(state, ec_d, eu_d, list(wl.w), lay, a_t[i], a_n[i], eta, 5, i + 1)
        z = sampler.noise(5, i + 1, idx) if eta else 0.0
        x = ddim.ddim_cfg_step_eps(x, ec.astype(np.float64), eu.astype(np.float64), w, a_t[i], a_n[i], eta, z)
        got = state.view(lay.n_maps, 2016).cpu().numpy()
        assert normwise_err(got, x) <= STATE_RTOL, f"step {i}"


def test_eps_step_chain_projection():
    torch, dev = torch_dev()
    wl = Workload("eps_chain", "", 8, 2, 6, 4, 12, 52, (50,), 1.0, (0.0, 1.0), None, 8)
    lay = layout_of(wl)
    say("eps step, two chains of 4 tiles, fused projection + discrepancy")
    ec, eu = _eps_inputs(lay.n_maps, 2)
    ec_d, eu_d = torch.from_numpy(ec).to(dev), torch.from_numpy(eu).to(dev)
    state = torch.empty(lay.n_maps * 2016, dtype=torch.float32, device=dev)
    pc.pc_init_state(state, lay, 9)
    x0 = state.view(lay.n_maps, 2016).cpu().numpy().astype(np.float64)
    pre = torch.empty(lay.n_seams * lay.n_guidance * lay.n_traj, dtype=torch.float32, device=dev)
    a_t, a_n = pc.pc_ddim_schedule(50)
    i = 20
    pc.pc_ddim_cfg_step_eps(state, ec_d, eu_d, list(wl.w), lay, a_t[i], a_n[i], 1.0, 9, i + 1, project_seams=True,
                            pre_disc=pre)
    got = state.view(lay.n_maps, 2016).cpu().numpy()
    idx = np.arange(lay.n_maps)
    w = np.asarray(wl.w)[(idx // wl.n_traj) % wl.n_guidance][:, None]
    stepped = ddim.ddim_cfg_step_eps(x0, ec.astype(np.float64), eu.astype(np.float64), w, a_t[i], a_n[i], 1.0,
                                     sampler.noise(9, i + 1, idx))
    G, S, L = wl.n_guidance, wl.n_traj, wl.chain_len
    pre_np = pre.cpu().numpy()
    for c in range(2):
        for g in range(G):
            for s in range(S):
                rows = [map_index(wl, c * L + k, g, s) for k in range(L)]
                col = stepped[rows][:, None, :]
                want_pre = seam.discrepancy_rms(col, 12)[:, 0]
                want = seam.project(col, 12)[:, 0, :]
                assert normwise_err(got[rows], want) <= STATE_RTOL
                assert np.all(seam.discrepancy_rms(got[rows][:, None, :].astype(np.float64), 12) == 0.0)
                gp = pre_np[[(c * (L - 1) + j) * G * S + g * S + s for j in range(L - 1)]]
                assert np.allclose(gp, want_pre, rtol=1e-5, atol=2e-5 * max(1.0, np.abs(col).max()))


def test_cosine_ddpm_chain_matches_oracle():
    # 1000 stride-1 steps with eta = 1 on the cosine schedule: the DDPM ancestral sampler
    torch, dev = torch_dev()
    wl = Workload("ddpm", "", 2, 2, 3, 1, 0, 0, (1000,), 1.0, (0.0, 1.0), None, 10)
    lay = layout_of(wl)
    say("cosine-schedule DDPM run, 1000 steps")
    refs = upload_refs(wl, 0)
    a_t, a_n = pc.pc_ddim_schedule_cosine(1000)
    state = torch.empty(lay.n_maps * 2016, dtype=torch.float32, device=dev)
    pc.pc_init_state(state, lay, 3)
    record = {1, 500, 999, 1000}
    rec = {}
    for i in range(1000):
        pc.pc_ddim_cfg_step(state, refs[2], refs[3], list(wl.w), lay, a_t[i], a_n[i], 1.0, 3, i + 1)
        if i + 1 in record:
            rec[i + 1] = state.view(lay.n_maps, 2016).cpu().numpy()
    idx = np.arange(lay.n_maps)
    r = idx // (wl.n_guidance * wl.n_traj)
    g = (idx // wl.n_traj) % wl.n_guidance
    ab = schedule.alpha_bar_from_betas(schedule.betas_cosine())
    x = sampler.noise(3, 0, idx)
    x0c, x0u = refs[0].astype(np.float64)[r], refs[1].astype(np.float64)[r]
    w = np.asarray(wl.w)[g][:, None]
    for i, (a, an) in enumerate(schedule.ddim_pairs(1000, ab=ab)):
        x = ddim.ddim_cfg_step(x, x0c, x0u, w, a, an, 1.0, sampler.noise(3, i + 1, idx))
        if i + 1 in record:
            assert normwise_err(rec[i + 1], x) <= STATE_RTOL, f"step {i + 1}"
