"""Launches split into several dispatches.

One dispatch holds at most 2^32 - 1 work-items, so grids beyond that are launched as
consecutive slices of the same grid.  Two checks:
  * every entry point gives bitwise the same result when the per-dispatch cap is lowered
    (pc_set_max_dispatch_items) so that small inputs are split into many slices;
  * a slab of 2^24 maps (135 GB of state), one map beyond what one dispatch of the
    independent-map step covers, takes x_T and one guided step that match the oracle on
    maps sampled on both sides of the slice boundary and at the ends.
"""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import STATE_RTOL, normwise_err, say, torch_dev
from oracle import ddim, sampler, schedule
from workloads import Workload, get, reference_maps

pytestmark = pytest.mark.gpu

CAPS = [1024, 3 * 512, 5 * 256 + 64]


@pytest.fixture
def capped():
    """Sets a dispatch cap for the test and always restores the hardware limit."""
    yield pc.pc_set_max_dispatch_items
    pc.pc_set_max_dispatch_items(0)


def _refs(torch, dev, R, seed):
    rng = np.random.default_rng(seed)
    x0c = torch.as_tensor(rng.uniform(0.5, 20.0, (R, 2016)).astype(np.float32), device=dev)
    x0u = torch.as_tensor(rng.uniform(0.5, 20.0, (R, 2016)).astype(np.float32), device=dev)
    return x0c.reshape(-1), x0u.reshape(-1)


@pytest.mark.parametrize("cap", CAPS)
def test_independent_entry_points_split_bitwise(capped, cap):
    torch, dev = torch_dev()
    lay = pc.PCLayout(3, 2, 37)   # 222 maps: 111 two-map workgroups, 222 one-map ones, 56 fill ones
    say(f"split independent maps, cap {cap}")
    x0c, x0u = _refs(torch, dev, lay.n_regions, 1)
    w = [0.0, 1.0]
    n = lay.n_maps * 2016
    gen = torch.Generator(device=dev).manual_seed(3)
    eps_c = torch.randn(n, generator=gen, device=dev)
    eps_u = torch.randn(n, generator=gen, device=dev)

    def run():
        out = {}
        s = torch.empty(n, dtype=torch.float32, device=dev)
        pc.pc_init_state(s, lay, 11)
        out["x_T"] = s.clone()
        pc.pc_ddim_cfg_step_eps(s, eps_c, eps_u, w, lay, 0.3, 0.5, 1.0, 11, 1)
        out["eps_step"] = s.clone()
        pc.pc_ddim_sample(s, x0c, x0u, w, lay, 50, 1.0, 11)
        out["sample"] = s.clone()
        words = torch.empty(n, dtype=torch.int32, device=dev)
        pc.pc_philox_fill(words, lay, 11, 7)
        out["words"] = words
        coords = torch.empty(lay.n_maps * 64 * 3, dtype=torch.float32, device=dev)
        ev = torch.empty(lay.n_maps * 3, dtype=torch.float32, device=dev)
        pc.pc_mds_recover(s, coords, ev)
        out["coords"], out["eig"] = coords, ev
        torch.cuda.synchronize()
        return out

    base = run()
    capped(cap)
    split = run()
    for k in base:
        assert torch.equal(base[k], split[k]), k


@pytest.mark.parametrize("cap", CAPS)
def test_chain_entry_points_split_bitwise(capped, cap):
    torch, dev = torch_dev()
    lay = pc.PCLayout(10, 2, 13, 5, 12)   # two chains of five tiles
    say(f"split chains, cap {cap}")
    x0c, x0u = _refs(torch, dev, lay.n_regions, 2)
    w = [0.0, 1.0]
    n = lay.n_maps * 2016
    n_seam_cols = lay.n_seams * lay.n_guidance * lay.n_traj

    def run():
        out = {}
        s = torch.empty(n, dtype=torch.float32, device=dev)
        pc.pc_ddim_sample(s, x0c, x0u, w, lay, 50, 1.0, 4, project_every=1)   # x_T drawn by the first step
        out["sample"] = s.clone()
        pc.pc_init_state(s, lay, 4)
        disc = torch.empty(n_seam_cols, dtype=torch.float32, device=dev)
        pc.pc_ddim_cfg_step(s, x0c, x0u, w, lay, 0.3, 0.5, 1.0, 4, 1, project_seams=False, pre_disc=disc)
        out["pre_disc"] = disc
        out["unprojected"] = s.clone()
        rms = torch.empty(n_seam_cols, dtype=torch.float32, device=dev)
        summ = torch.empty(2, dtype=torch.float32, device=dev)
        pc.pc_seam_discrepancy(s, lay, rms, summ)
        out["rms"], out["summary"] = rms, summ
        ma = torch.empty(lay.n_seams * lay.n_guidance, dtype=torch.float32, device=dev)
        pc.pc_seam_mean_abs(s, lay, ma)
        out["mean_abs"] = ma
        pc.pc_seam_project(s, lay)
        out["projected"] = s.clone()
        coords = torch.empty(lay.n_maps * 64 * 3, dtype=torch.float32, device=dev)
        pc.pc_mds_recover(out["sample"], coords)
        n_beads = (lay.chain_len - 1) * (64 - lay.overlap) + 64
        chain = torch.empty(2 * lay.n_guidance * lay.n_traj * n_beads * 3, dtype=torch.float32, device=dev)
        resid = torch.empty(n_seam_cols, dtype=torch.float32, device=dev)
        pc.pc_kabsch_stitch(coords, lay, chain, resid)
        out["chain"], out["resid"] = chain, resid
        chain_p, resid_p = torch.empty_like(chain), torch.empty_like(resid)
        pc.pc_kabsch_stitch_proper(coords, lay, chain_p, resid_p)
        out["chain_proper"], out["resid_proper"] = chain_p, resid_p
        torch.cuda.synchronize()
        return out

    base = run()
    capped(cap)
    split = run()
    for k in base:
        assert torch.equal(base[k], split[k]), k


def test_slab_of_2p24_maps_one_step():
    """2^24 maps = 65,536 regions x 2 weights x 128 trajectories: the independent-map step needs
    8,388,608 two-map workgroups, one more than a dispatch of 512-lane workgroups holds, so it runs
    as two dispatches.  References: the genome-wide slab's 2,658 seeded pairs, region r taking pair
    r mod 2,658."""
    torch, dev = torch_dev()
    base = get("genome_slab")
    wl = Workload("slab_2p24", "", 65536, 2, 128, 1, 0, 0, (50,), 1.0, (0.0, 1.0), None, base.family)
    seed = 2
    say("slab of 2^24 maps (135 GB): x_T and one guided step, sampled maps")
    x0c_s, x0u_s = reference_maps(base, seed)
    reg = np.arange(wl.n_regions) % base.n_regions
    x0c = torch.as_tensor(x0c_s, device=dev)[torch.as_tensor(reg, device=dev)].contiguous()
    x0u = torch.as_tensor(x0u_s, device=dev)[torch.as_tensor(reg, device=dev)].contiguous()
    lay = pc.PCLayout(wl.n_regions, wl.n_guidance, wl.n_traj)
    assert lay.n_maps == 1 << 24
    state = torch.empty(lay.n_maps * 2016, dtype=torch.float32, device=dev)
    pc.pc_init_state(state, lay, seed)
    a_t, a_n = pc.pc_ddim_schedule(50)
    pc.pc_ddim_cfg_step(state, x0c, x0u, list(wl.w), lay, a_t[0], a_n[0], wl.eta, seed, 1)
    # the second dispatch starts at logical workgroup 8,388,607 = maps 16,777,214 and 16,777,215
    rng = np.random.default_rng(9)
    idx = np.unique(np.concatenate([[0, 1, 16777212, 16777213, 16777214, 16777215, 8388606, 8388607],
                                    rng.choice(lay.n_maps, 24, replace=False)]))
    got = state.view(lay.n_maps, 2016)[torch.as_tensor(idx, device=dev)].cpu().numpy()
    del state, x0c, x0u
    torch.cuda.empty_cache()
    G, S = wl.n_guidance, wl.n_traj
    r = (idx // (G * S)) % base.n_regions
    g = (idx // S) % G
    x_t = sampler.noise(seed, 0, idx)
    (a, an), = schedule.ddim_pairs(50)[:1]
    want = ddim.ddim_cfg_step(x_t, x0c_s[r].astype(np.float64), x0u_s[r].astype(np.float64),
                              np.asarray(wl.w)[g].reshape(-1, 1), a, an, wl.eta, sampler.noise(seed, 1, idx))
    err = normwise_err(got, want)
    say(f"  worst normwise error {err:.3e}")
    assert err <= STATE_RTOL
