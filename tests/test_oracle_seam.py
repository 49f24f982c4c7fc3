"""Pins for the oracle's tiling geometry, seam projection and discrepancy."""

import json
import math
import os

import numpy as np
import pytest

from oracle import layout, sampler, schedule, seam
from workloads import get, reference_maps

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "chr22_tiling.json")))


def test_chr22_geometry_from_the_pages():
    n, o = GOLD["beads_per_region"], GOLD["overlap_beads"]
    stride = n - o
    assert (GOLD["chr22_tiles"] - 1) * stride + n == GOLD["chr22_monomers"]
    assert GOLD["chr22_tiles"] - 1 == GOLD["chr22_seams"]
    wl = get("chr22_chain")
    assert (wl.chain_len, wl.overlap, wl.stride, wl.chain_beads) == (GOLD["chr22_tiles"], o, stride,
                                                                     GOLD["chr22_monomers"])
    li, ri = seam.seam_pairs(o)
    assert len(li) == len(ri) == o * (o - 1) // 2 == 66
    # beads of a middle tile that lie in neither overlap
    lo, hi = GOLD["non_overlap_beads"]
    inner = [b for b in range(n) if b >= o and b < n - o]
    assert (inner[0], inner[-1]) == (lo, hi)


def test_seam_index_map_brute_force():
    # enumerate global bead pairs that lie in both tiles k and k+1, and locate them in each tile's
    # packed map by searching numpy's triu order (independent of layout.idx)
    n, o = 64, 12
    stride = n - o
    iu, ju = np.triu_indices(n, 1)
    where = {(int(i), int(j)): e for e, (i, j) in enumerate(zip(iu, ju))}
    for k in (0, 5, 30):
        a0, b0 = k * stride, (k + 1) * stride
        shared = sorted(set(range(a0, a0 + n)) & set(range(b0, b0 + n)))
        assert len(shared) == o
        left, right = [], []
        for x in range(len(shared)):
            for y in range(x + 1, len(shared)):
                g1, g2 = shared[x], shared[y]
                left.append(where[(g1 - a0, g2 - a0)])
                right.append(where[(g1 - b0, g2 - b0)])
        li, ri = seam.seam_pairs(o)
        assert list(li) == left and list(ri) == right


def test_right_seam_is_the_packed_tail():
    li, _ = seam.seam_pairs(12)
    assert list(li) == list(range(1950, 2016))
    assert layout.idx(52, 53) == 1950 and layout.idx(62, 63) == 2015


def _chain_states(L=5, B=3, seed=0):
    return np.random.default_rng(seed).uniform(0, 30, (L, B, 2016))


def test_projection_invariants():
    x = _chain_states()
    y = seam.project(x, 12)
    li, ri = seam.seam_pairs(12)
    assert np.all(seam.discrepancy_rms(y, 12) == 0.0)
    assert np.array_equal(seam.project(y, 12), y)  # idempotent, bitwise
    mask = np.ones((x.shape[0], 2016), dtype=bool)
    mask[:-1, li] = False
    mask[1:, ri] = False
    for k in range(x.shape[0]):
        assert np.array_equal(x[k][:, mask[k]], y[k][:, mask[k]])  # only seam entries change
    for k in range(x.shape[0] - 1):
        assert np.allclose(y[k][:, li] + y[k + 1][:, ri], x[k][:, li] + x[k + 1][:, ri], rtol=1e-15)
    one = x[:1]
    assert np.array_equal(seam.project(one, 12), one)


def test_discrepancy_matches_unpacked_blocks():
    x = _chain_states(L=3, B=2, seed=4)
    d = seam.discrepancy_rms(x, 12)
    for k in range(2):
        for b in range(2):
            left = layout.unpack(x[k, b])[52:, 52:]
            right = layout.unpack(x[k + 1, b])[:12, :12]
            iu = np.triu_indices(12, 1)
            diff = (left - right)[iu]
            assert d[k, b] == pytest.approx(math.sqrt(np.mean(diff ** 2)), rel=1e-14)
            # the unpacked blocks are symmetric, and projection makes them equal
            y = seam.project(x, 12)
            assert np.array_equal(layout.unpack(y[k, b])[52:, 52:], layout.unpack(y[k + 1, b])[:12, :12])


def test_mean_abs_discrepancy_small_case():
    x = np.zeros((2, 2, 2016))
    li, ri = seam.seam_pairs(12)
    x[0][:, li] = [[1.0], [3.0]]  # sample mean 2 on the left copy
    x[1][:, ri] = 0.5
    assert seam.discrepancy_mean_abs(x, 12)[0] == pytest.approx(1.5)


@pytest.mark.slow
def test_pre_projection_discrepancy_is_two_sigma_squared():
    # After a projection both copies of a seam pair agree, the stand-in step is elementwise and the
    # references agree on the seam, so before the next projection the copies differ only by
    # sigma (z_k - z_{k+1}): mean square 2 sigma^2.  At the last step sigma = 0.
    wl = get("chr22_chain")
    x0c, x0u = reference_maps(wl, 0)
    L, B = 6, 64
    tids = np.arange(L * B).reshape(L, B)
    _, _, pre, post = sampler.run_chain(x0c[:L], x0u[:L], np.tile([0.0, 1.0], B // 2), tids, seed=5,
                                        n_steps=50, eta=1.0, overlap=12)
    assert np.all(post == 0.0)
    pairs = schedule.ddim_pairs(50)
    for i in (1, 10, 30, 48):
        sig = schedule.ddim_sigma(*pairs[i], 1.0)
        ms = np.mean(pre[i] ** 2)
        assert ms == pytest.approx(2 * sig * sig, rel=0.05)
    assert np.all(pre[-1] == 0.0)
