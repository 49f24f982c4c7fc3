"""GPU parity of the noise source: Philox words bit-exact, normals within float32
transcendental error, x_T equal to slot 0."""

import numpy as np
import pytest

import tiled_genome_diffusion_amd as pc
from oracle import normals, philox
from gpu_util import say, torch_dev

pytestmark = pytest.mark.gpu

# |z_gpu - z_oracle|: float32 log, sqrt and sincospi on radii up to sqrt(48 ln 2) ~ 5.77;
# a few ulp of each factor gives < 2e-6.
NORMAL_ATOL = 4e-6


@pytest.mark.parametrize("seed,slot", [(0, 0), (1, 1), (2, 37), (0xDEADBEEF12345678, 1000)])
def test_philox_words_bit_exact(seed, slot):
    torch, dev = torch_dev()
    lay = pc.PCLayout(3, 2, 5)   # 30 maps, ragged against the 4-map fill blocks
    say(f"philox words seed={seed} slot={slot}")
    out = torch.empty(lay.n_maps * 2016, dtype=torch.int32, device=dev)
    pc.pc_philox_fill(out, lay, seed, slot)
    got = out.cpu().numpy().view(np.uint32).reshape(lay.n_maps, 2016)
    want = philox.map_words(seed, np.arange(lay.n_maps), slot)
    assert np.array_equal(got, want)


def test_philox_words_high_trajectory_ids():
    torch, dev = torch_dev()
    lay = pc.PCLayout(2658, 2, 100)   # the genome-wide slab, 531,600 maps
    say("philox words on the 531,600-map layout")
    out = torch.empty(lay.n_maps * 2016, dtype=torch.int32, device=dev)
    pc.pc_philox_fill(out, lay, 3, 50)
    rows = np.array([0, 1, 4095, 265_799, 531_598, 531_599])
    got = out.view(lay.n_maps, 2016)[torch.as_tensor(rows, device=dev)].cpu().numpy().view(np.uint32)
    assert np.array_equal(got, philox.map_words(3, rows, 50))
    del out
    torch.cuda.empty_cache()


def test_normals_and_initial_state():
    torch, dev = torch_dev()
    lay = pc.PCLayout(2, 2, 50)
    say("normals / init state")
    z = torch.empty(lay.n_maps * 2016, dtype=torch.float32, device=dev)
    x = torch.empty_like(z)
    for slot in (0, 7):
        pc.pc_normal_fill(z, lay, 11, slot)
        want = normals.words_to_normals(philox.map_words(11, np.arange(lay.n_maps), slot))
        got = z.cpu().numpy().reshape(lay.n_maps, 2016)
        assert np.abs(got - want).max() <= NORMAL_ATOL
    pc.pc_init_state(x, lay, 11)
    pc.pc_normal_fill(z, lay, 11, 0)
    assert torch.equal(x, z)
