"""Host-side logic of bench.py (no GPU): the one-GPU refusal, the counter-to-traffic
conversion, the source-hash guard on stored traffic figures, and the oracle baseline's
JSON fields."""

import csv
import hashlib
import importlib.util
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _run(*args, timeout=600):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=timeout, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writerows(rows)


def test_traffic_summary_scales_counters_by_the_copy(tmp_path):
    # single_region: 16 maps; the copy moves 16 * 2016 * 4 = 129,024 B (126 KiB)
    copy_kib = 16 * 2016 * 4 / 1024.0
    step = "void pc::(anonymous namespace)::k_step_indep<2, true, true, false>(float*)"
    copy = "__amd_rocclr_copyBuffer"
    _write_counters(tmp_path / "copy_FETCH_SIZE", [[copy, "FETCH_SIZE", copy_kib / 2]])
    _write_counters(tmp_path / "copy_WRITE_SIZE", [[copy, "WRITE_SIZE", copy_kib]])
    # three dispatches: the x_T-drawing one reads almost nothing; the median is taken
    _write_counters(tmp_path / "slab_FETCH_SIZE", [[step, "FETCH_SIZE", v] for v in (1.0, 70.0, 71.0)])
    _write_counters(tmp_path / "slab_WRITE_SIZE", [[step, "WRITE_SIZE", v] for v in (126.0, 126.0, 126.0)])
    out = tmp_path / "traffic.json"
    r = _run("--workload", "single_region", "--traffic-summary", str(tmp_path), "--traffic-out", str(out))
    assert r.returncode == 0, r.stderr
    d = json.loads(out.read_text())
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["fetch_size_kib_per_launch"] == 70.0 and d["launches"] == 3
    assert d["traffic_bytes_per_launch"] == pytest.approx(70.0 * 1024 * 2 + 126.0 * 1024)
    assert d["algorithmic_read_bytes"] == 16 * 8064 + 1 * 16128 and d["algorithmic_write_bytes"] == 16 * 8064


def test_stored_traffic_is_used_only_while_the_source_is_unchanged(tmp_path):
    bench = _bench_module()
    h = hashlib.sha256()
    for rel in bench.STEP_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    rec = {"workload": "single_region", "source_files": bench.STEP_SOURCES, "source_sha256": h.hexdigest(),
           "traffic_bytes_per_launch": 1234.0, "kernel": "k_step_indep<2, true, true, false>"}
    (tmp_path / "a_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("single_region", str(tmp_path)) == (1234.0, rec["kernel"])
    assert bench.measured_traffic("genome_slab", str(tmp_path)) == (None, None)
    rec["source_sha256"] = "0" * 64
    (tmp_path / "a_traffic.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("single_region", str(tmp_path)) == (None, None)


def test_cpu_only_reports_the_oracle_baseline_fields():
    r = _run("--workload", "single_region", "--cpu-only", "--cpu-seconds", "0.2", "--cpu-procs", "2",
             "--jacobi-maps", "2")
    assert r.returncode == 0, r.stderr
    d = json.loads(r.stdout.strip().splitlines()[-1])
    cb = d["cpu_baseline"]
    assert cb["value"] > 0 and cb["unit"] == "trajectory-steps/s" and cb["cores"] == 1 and cb["kind"] == "oracle"
    assert "16 of 16 maps" in cb["sample"]
    assert cb["jacobi_mds"]["maps"] == 2 and cb["jacobi_mds"]["maps_per_s"] > 0
    par = d["cpu_baseline_parallel"]
    assert par["cores"] == 2 and par["value"] > 0


def test_probe_library_exports_its_probes():
    """The HBM-ceiling probes are built beside libpc.so, export their three entry points, and are
    not part of include/pc.h."""
    import re

    from tiled_genome_diffusion_amd import build as libbuild

    if not os.path.exists(libbuild.CEILING_LIB):
        pytest.fail("libpc_ceiling.so is not built (python -m tiled_genome_diffusion_amd.build)")
    out = subprocess.run(["nm", "-D", "--defined-only", libbuild.CEILING_LIB], capture_output=True, text=True,
                         check=True).stdout
    names = set(re.findall(r"\bT (pcc_\w+)", out))
    assert names == {"pcc_probe_rmw", "pcc_probe_read", "pcc_probe_write"}
    with open(os.path.join(ROOT, "include", "pc.h")) as f:
        assert "pcc_" not in f.read()
    bench = _bench_module()
    assert bench.probe_lib() is not None
