"""Seeded random layouts through the whole-loop entry point, against the oracle.

Each case draws a small layout (regions or chains of tiles, guidance weights,
trajectories, overlap, projection interval), a step count, eta and weights
from a fixed generator, runs pc_ddim_sample on the GPU (x_T drawn in the
first step for independent maps, filled for seam-projecting chains) and
compares every final map with the float64 oracle, then MDS of a few of them.
The cases are fixed when the module is imported, so a failure names its case.
"""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import DIST_RTOL, STATE_RTOL, layout_of, normwise_err, rel_dist_err, say, torch_dev, upload_refs
from oracle import mds, sampler
from workloads import Workload

pytestmark = pytest.mark.gpu


def _cases(n=12, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        chain = k % 2 == 1
        L = int(rng.integers(2, 7)) if chain else 1
        R = L * int(rng.integers(1, 3)) if chain else int(rng.integers(1, 6))
        G = int(rng.integers(1, 5))
        S = int(rng.integers(1, 12))
        O = int(rng.integers(2, 33)) if chain else 0
        K = int(rng.integers(0, 4)) if chain else 0
        n_steps = int(rng.choice([10, 20, 25, 40]))
        eta = float(rng.choice([0.0, 0.3, 1.0]))
        w = tuple(float(v) for v in np.round(rng.uniform(-1.0, 3.0, G), 3))
        out.append((k, R, G, S, L, O, K, n_steps, eta, w))
    return out


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[0]}-R{c[1]}G{c[2]}S{c[3]}L{c[4]}O{c[5]}K{c[6]}")
def test_random_layout_matches_oracle(case):
    k, R, G, S, L, O, K, n_steps, eta, w = case
    torch, dev = torch_dev()
    wl = Workload(f"random{k}", "", R, G, S, L, O, 64 - O if L > 1 else 0, (n_steps,), eta, w, None, 20 + k)
    seed = 1000 + k
    say(f"random layout {case}")
    refs = upload_refs(wl, seed)
    lay = layout_of(wl)
    state = torch.full((lay.n_maps * 2016,), float("nan"), dtype=torch.float32, device=dev)
    pc.pc_ddim_sample(state, refs[2], refs[3], list(w), lay, n_steps, eta, seed, project_every=K)
    got = state.view(lay.n_maps, 2016).cpu().numpy()

    if L == 1:
        idx = np.arange(lay.n_maps)
        r, g = idx // (G * S), (idx // S) % G
        want, _ = sampler.run_independent(refs[0][r], refs[1][r], np.asarray(w)[g], idx, seed, n_steps, eta)
        want = want.reshape(lay.n_maps, 2016)
    else:
        want = np.empty((lay.n_maps, 2016))
        cols = [(g, s) for g in range(G) for s in range(S)]
        for c in range(R // L):
            tids = np.array([[((c * L + t) * G + g) * S + s for (g, s) in cols] for t in range(L)])
            fin, _, _, _ = sampler.run_chain(refs[0][c * L:(c + 1) * L], refs[1][c * L:(c + 1) * L],
                                             np.array([w[g] for (g, _) in cols]), tids, seed, n_steps, eta, O,
                                             project_every=K if K > 0 else n_steps + 1)
            want[tids.reshape(-1)] = fin.reshape(-1, 2016)
    assert normwise_err(got, want) <= STATE_RTOL

    # MDS of final maps whose weight lies in [0, 1] (the final maps are the weighted mixtures of the
    # two references, and extrapolated mixtures are far from Euclidean)
    gidx = (np.arange(lay.n_maps) // S) % G
    ok = np.nonzero((np.asarray(w)[gidx] >= 0.0) & (np.asarray(w)[gidx] <= 1.0))[0]
    if ok.size == 0:
        return
    sample = ok[np.unique(np.linspace(0, ok.size - 1, 6).astype(int))]
    coords = torch.empty(len(sample) * 64 * 3, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(state.view(lay.n_maps, 2016)[torch.as_tensor(sample, device=dev)].contiguous(), coords,
                      max_iters=256)
    coords = coords.view(len(sample), 64, 3).cpu().numpy()
    for c, m in zip(coords, got[sample]):
        o, _ = mds.classical_mds(m.astype(np.float64))
        assert rel_dist_err(mds.coords_distances(c), mds.coords_distances(o)) <= DIST_RTOL
