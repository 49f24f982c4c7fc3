"""The bandwidth probes bench.py measures the HBM ceiling with (libpc_ceiling.so) move every
element: the read-modify-write computes a x + b in place, the write stores its value everywhere,
and the read leaves its sink alone unless a lane's sum equals the sentinel."""

import numpy as np
import pytest

from gpu_util import say, torch_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_maps", [1, 7, 1500])
def test_probes_touch_every_element(n_maps):
    import ctypes
    import importlib.util
    import os

    torch, dev = torch_dev()
    say(f"bandwidth probes, {n_maps} maps")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("bench_probe", os.path.join(root, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    lib = bench.probe_lib()
    st = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    x = torch.as_tensor(np.random.default_rng(n_maps).standard_normal(n_maps * 2016).astype(np.float32), device=dev)
    want = torch.addcmul(torch.full_like(x, 1.0), x, torch.full_like(x, 2.0))   # 2 x + 1, one rounding
    assert lib.pcc_probe_rmw(ctypes.c_void_p(x.data_ptr()), n_maps, 2.0, 1.0, st) == 0
    sink = torch.full((1,), -7.0, dtype=torch.float32, device=dev)
    assert lib.pcc_probe_read(ctypes.c_void_p(x.data_ptr()), n_maps, float("nan"), ctypes.c_void_p(sink.data_ptr()),
                              st) == 0
    torch.cuda.synchronize()
    assert torch.equal(x, want)
    assert float(sink[0]) == -7.0
    assert lib.pcc_probe_write(ctypes.c_void_p(x.data_ptr()), n_maps, 0.25, st) == 0
    torch.cuda.synchronize()
    assert bool((x == 0.25).all())
