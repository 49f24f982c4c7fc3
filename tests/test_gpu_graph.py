"""The whole-chain entry point enqueues only kernels (no memsets, no host
synchronisation), so callers can capture it in a HIP graph: every replay must
reproduce the eager result bitwise."""

import pytest

import tiled_genome_diffusion_amd as pc
from gpu_util import layout_of, say, torch_dev, upload_refs
from workloads import get

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["region_ensemble", "chr22_chain"])
def test_graph_replays_match_eager(name):
    torch, dev = torch_dev()
    wl = get(name)
    lay = layout_of(wl)
    say(f"graph capture of the whole chain: {name}")
    refs = upload_refs(wl, 0)
    project = 1 if wl.chain_len > 1 else 0
    eager = torch.empty(lay.n_maps * 2016, dtype=torch.float32, device=dev)
    pc.pc_ddim_sample(eager, refs[2], refs[3], list(wl.w), lay, 50, wl.eta, 0, project_every=project)
    coords_e = torch.empty(lay.n_maps * 192, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(eager, coords_e)
    torch.cuda.synchronize()

    state = torch.empty_like(eager)
    coords = torch.empty_like(coords_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up outside the capture, on the capture stream
        pc.pc_ddim_sample(state, refs[2], refs[3], list(wl.w), lay, 50, wl.eta, 0, project_every=project)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pc.pc_ddim_sample(state, refs[2], refs[3], list(wl.w), lay, 50, wl.eta, 0, project_every=project)
        pc.pc_mds_recover(state, coords)
    for rep in range(4):
        state.fill_(float("nan"))          # eager work between replays
        coords.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, eager), f"replay {rep}"
        assert torch.equal(coords, coords_e), f"replay {rep}"
