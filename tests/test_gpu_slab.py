"""The genome-wide slab at full size (2658 regions x 2 weights x 100 trajectories,
531,600 maps, 4.3 GB of state) in the launch configuration the benchmark
times, checked on sampled maps against the oracle."""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import (DIST_RTOL, STATE_RTOL, layout_of, normwise_err, rel_dist_err, run_steps, say, torch_dev,
                      upload_refs)
from oracle import mds, sampler
from workloads import get

pytestmark = pytest.mark.gpu


def test_genome_slab_sampled():
    torch, dev = torch_dev()
    wl = get("genome_slab")
    seed = 1
    say("genome_slab: 531,600 maps, 64 sampled, steps 1/10/25/50")
    refs = upload_refs(wl, seed)
    rng = np.random.default_rng(42)
    idx = np.sort(np.concatenate([[0, wl.n_maps - 1], rng.choice(wl.n_maps, 62, replace=False)]))
    record = {1, 10, 25, 50}
    rec, state, _ = run_steps(wl, seed, 50, idx, record, refs=refs)
    G, S = wl.n_guidance, wl.n_traj
    r = idx // (G * S)
    g = (idx // S) % G
    _, orec = sampler.run_independent(refs[0][r], refs[1][r], np.asarray(wl.w)[g], idx, seed, 50, wl.eta,
                                      record=record)
    for s in sorted(record):
        err = normwise_err(rec[s], orec[s])
        say(f"  step {s}: worst normwise error {err:.3e}")
        assert err <= STATE_RTOL
    # the whole-loop entry point reproduces the step loop bitwise
    lay = layout_of(wl)
    s2 = torch.empty_like(state)
    pc.pc_ddim_sample(s2, refs[2], refs[3], list(wl.w), lay, 50, wl.eta, seed)
    assert torch.equal(s2, state)
    del s2
    # MDS over all final maps; sampled maps against the oracle
    coords = torch.empty(wl.n_maps * 64 * 3, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(state, coords)
    got = coords.view(wl.n_maps, 64, 3)[torch.as_tensor(idx, device=dev)].cpu().numpy()
    for c, m in zip(got, rec[50]):
        o, _ = mds.classical_mds(m.astype(np.float64))
        assert rel_dist_err(mds.coords_distances(c), mds.coords_distances(o)) <= DIST_RTOL
    del state, coords
    torch.cuda.empty_cache()
