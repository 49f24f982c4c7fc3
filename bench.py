"""Benchmark of the hot path on one MI355X.

One step = one full pass over a batch of synthetic input: x_T for every map,
the workload's guided DDIM steps (with seam projection for chains) and
classical MDS of every final map.  Default workload: the genome-wide slab,
2658 regions x 2 guidance weights x 100 trajectories = 531,600 maps (4.3 GB of
float32 state), 50 steps, eta = 1.

Prints one JSON line.  `value` is trajectory-steps per second of the whole
pass; `roofline` describes the DDIM step kernel (HBM-bound), timed with HIP
events on the stream it runs on; `cpu_baseline` times the float64 oracle on a
bounded sample of the same workload on the host.
"""

from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
STEP_BYTES_PER_MAP = 2016 * 4 * 2   # read + write of one packed map per DDIM step
REF_BYTES_PER_REGION = 2016 * 4 * 2  # conditional + unconditional reference, once per region per step
FP32_PEAK_TFLOPS = 157.3       # MI355X FP32 vector, published (counts packed-FP32 instructions)
# Non-packed FP32 vector peak: 256 CUs x 4 SIMDs x 16 lanes x 2 flops (FMA) x 2.4 GHz.  The library
# is built with packed-FP32 instructions disabled, so this is the ceiling its vector code can reach.
FP32_NONPACKED_PEAK_TFLOPS = 78.6
MDS_BYTES_PER_MAP = 2016 * 4 + 64 * 3 * 4   # packed map read + coordinates written (eigenvalues optional)
# Algorithmic flops of classical MDS on one map along the path a Euclidean map takes (two
# products B Q and one Rayleigh-Ritz step): squaring and double centring 16,384; the two
# 64x64x4 products 65,536; Gram-Schmidt of four columns 2,304; H = Q^T Z 1,280; Ritz vectors
# and residuals 4,864; output 192.
MDS_FLOPS_PER_MAP = 16384 + 65536 + 2304 + 1280 + 4864 + 192


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=6, help="timed passes")
    p.add_argument("--warmup", type=int, default=None,
                   help="untimed passes (default: 1 for states of 1 GB and more, else 30: passes of a few "
                        "milliseconds do not settle the GPU's clocks)")
    p.add_argument("--workload", default="genome_slab")
    p.add_argument("--n-steps", type=int, default=0, help="DDIM steps (default: the workload's first)")
    p.add_argument("--seed", type=int, default=0, help="seed of the ablation and cpu baseline")
    p.add_argument("--seeds", default="0,1,2",
                   help="base seeds the timed passes cycle through (inputs and noise); per-seed rates are reported")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target duration of the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-procs", type=int, default=0,
                   help="with --cpu-only: also time the oracle in this many processes over disjoint blocks")
    p.add_argument("--cpu-only", action="store_true",
                   help="no GPU: print only the oracle baseline of the workload (one JSON line)")
    p.add_argument("--eps-buffers", action="store_true",
                   help="step with noise predictions read from buffers (the interface of a trained denoiser) "
                        "instead of the point-mass stand-in: 16 B per element-step instead of 8")
    p.add_argument("--graph", action="store_true",
                   help="capture one pass in a HIP graph and time graph replays (for launch-bound small workloads)")
    p.add_argument("--sync-ablation", default="",
                   help="comma-separated projection intervals K (0 = never) for a sync-frequency ablation on a "
                        "chain workload; prints one JSON line with a row per K")
    p.add_argument("--chain-kernels", action="store_true",
                   help="on a chain workload: time the kernels off the step path (Kabsch stitching, the seam "
                        "discrepancies, standalone projection) on the final state of one pass; one JSON line")
    p.add_argument("--traffic-summary", default="", metavar="PMC_DIR",
                   help="no GPU: turn the FETCH_SIZE / WRITE_SIZE counter runs under PMC_DIR (copy_<C>/ and "
                        "slab_<C>/ rocprofv3 csv output) into profiles/k_step_indep_<workload>_traffic.json")
    p.add_argument("--traffic-out", default="", metavar="PATH",
                   help="with --traffic-summary: write the JSON here instead of under profiles/")
    p.add_argument("--copy-only", action="store_true",
                   help="time a plain device-to-device copy of the workload's state size instead "
                        "(the calibration kernel for the HBM byte counters)")
    p.add_argument("--ceilings", action="store_true",
                   help="time the bandwidth probes (in-place read-modify-write, read-only and write-only "
                        "streams with the step kernel's access pattern) and the x_T fill on the workload's state; "
                        "one JSON line")
    p.add_argument("--seam-report", action="store_true",
                   help="on a chain workload: per-step seam discrepancy before projection (the fused "
                        "discrepancy output of the step) and after it (pc_seam_discrepancy), against the "
                        "closed-form expectation, and the step time with and without the discrepancy output")
    p.add_argument("--mds-inputs", action="store_true",
                   help="time MDS alone over the workload's map count on three kinds of input: the exact "
                        "final maps, the same with 1e-3 relative noise, and equal mixtures of two regions' maps "
                        "(not Euclidean); one JSON line")
    p.add_argument("--jacobi-maps", type=int, default=8,
                   help="maps the cpu baseline runs through the Jacobi MDS oracle (0.5 s each on one core)")
    return p.parse_args()


def measured_traffic(workload: str, directory: str = os.path.join(ROOT, "profiles")):
    """HBM bytes per step launch from the committed FETCH_SIZE/WRITE_SIZE counter runs
    (profiles/*_traffic.json), or None if none matches this workload or the kernel
    source has changed since the counters were taken."""
    for path in glob.glob(os.path.join(directory, "*_traffic.json")):
        with open(path) as f:
            d = json.load(f)
        if d.get("workload") != workload:
            continue
        h = hashlib.sha256()
        for rel in d["source_files"]:  # the files the counters were taken on
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        if h.hexdigest() == d["source_sha256"]:
            return d["traffic_bytes_per_launch"], d["kernel"]
    return None, None


STEP_SOURCES = ["tiled_genome_diffusion_amd/csrc/step.hip", "tiled_genome_diffusion_amd/csrc/stream.hpp",
                "tiled_genome_diffusion_amd/csrc/common.hpp", "tiled_genome_diffusion_amd/csrc/launch.hpp",
                "tiled_genome_diffusion_amd/csrc/dispatch.hpp"]


def traffic_summary(args, wl):
    """Scale the step kernel's FETCH_SIZE / WRITE_SIZE (KiB per dispatch, median over
    the dispatches) by what the same counters read for the plain copy of
    bench.py --copy-only, and store the result with the hash of the kernel source
    it was measured on."""
    import csv

    def per_kernel(run, counter):
        path = glob.glob(os.path.join(args.traffic_summary, f"{run}_{counter}", "*_counter_collection.csv"))[0]
        acc = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        # the median dispatch: the first step of a pass draws x_T instead of reading it, so
        # one dispatch in 49 of the step kernel reads no state
        return {k: (sorted(v)[len(v) // 2], len(v)) for k, v in acc.items()}

    copy_bytes = wl.n_maps * 2016 * 4
    scale = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        kib = max(per_kernel("copy", c).values())[0]   # the copy dispatch dominates the run
        scale[c] = (kib, copy_bytes / 1024.0 / kib)
    fetch, write = per_kernel("slab", "FETCH_SIZE"), per_kernel("slab", "WRITE_SIZE")
    name = max((k for k in fetch if "k_step_indep" in k), key=lambda k: fetch[k][1])   # the noisy-step form
    h = hashlib.sha256()
    for rel in STEP_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    rd = fetch[name][0] * 1024 * scale["FETCH_SIZE"][1]
    wr = write[name][0] * 1024 * scale["WRITE_SIZE"][1]
    def short(k):
        return k.replace("void ", "").replace("pc::(anonymous namespace)::", "").split("(")[0]

    out = {"kernel": short(name), "workload": wl.name,
           "source_files": STEP_SOURCES, "source_sha256": h.hexdigest(),
           "fetch_size_kib_per_launch": fetch[name][0], "write_size_kib_per_launch": write[name][0],
           "launches": fetch[name][1], "statistic": "median dispatch",
           "copy_fetch_size_kib": scale["FETCH_SIZE"][0], "copy_write_size_kib": scale["WRITE_SIZE"][0],
           "copy_bytes": copy_bytes, "fetch_scale": scale["FETCH_SIZE"][1], "write_scale": scale["WRITE_SIZE"][1],
           "traffic_bytes_per_launch": rd + wr, "fetch_bytes_per_launch": rd, "write_bytes_per_launch": wr,
           "algorithmic_read_bytes": wl.n_maps * 2016 * 4 + wl.n_regions * REF_BYTES_PER_REGION,
           "algorithmic_write_bytes": wl.n_maps * 2016 * 4}
    dest = args.traffic_out or os.path.join(ROOT, "profiles", f"k_step_indep_{wl.name}_traffic.json")
    with open(dest, "w") as f:
        json.dump(out, f, indent=1)
    for k in sorted(fetch):
        fr, wr_ = fetch[k][0], write.get(k, (float("nan"), 0))[0]
        print(f"| `{short(k)}` (median of {fetch[k][1]}) | {fr:,.0f} | {wr_:,.0f} | "
              f"{fr * 1024 * scale['FETCH_SIZE'][1]:,.0f} | {wr_ * 1024 * scale['WRITE_SIZE'][1]:,.0f} |")
    print(json.dumps(out, indent=1))


def copy_only(args, wl):
    """A plain copy of known size: the reference for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    n = wl.n_maps * 2016
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "ms": dt * 1e3,
                      "gbs": 2 * n * 4 / dt / 1e9, "workload": wl.name}), flush=True)


def probe_lib():
    """The bandwidth probes of libpc_ceiling.so (built beside libpc.so; not part of include/pc.h)."""
    import ctypes

    from tiled_genome_diffusion_amd import build as libbuild

    if not os.path.exists(libbuild.CEILING_LIB):
        raise SystemExit(f"{libbuild.CEILING_LIB} is not built (python -m tiled_genome_diffusion_amd.build)")
    lib = ctypes.CDLL(libbuild.CEILING_LIB)
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    lib.pcc_probe_rmw.argtypes = [vp, i64, f32, f32, vp]
    lib.pcc_probe_read.argtypes = [vp, i64, f32, vp, vp]
    lib.pcc_probe_write.argtypes = [vp, i64, f32, vp]
    for f in (lib.pcc_probe_rmw, lib.pcc_probe_read, lib.pcc_probe_write):
        f.restype = ctypes.c_int
    return lib


def hbm_probes(state, n_maps, stream, reps=5):
    """GB/s of the three probes over `state` (n_maps packed maps; overwritten), each the median
    of `reps` timings with HIP events on `stream`, after one untimed launch.  A timing spans one
    launch for states of 1 GB and more, and 20 back-to-back launches for smaller ones, whose
    launches last tens of microseconds: one launch between two events would also time the
    launch latency, which back-to-back launches of the step loop do not pay."""
    import ctypes

    import numpy as np
    import torch

    lib = probe_lib()
    ptr, st = ctypes.c_void_p(state.data_ptr()), ctypes.c_void_p(stream.cuda_stream)
    sink = torch.zeros(1, dtype=torch.float32, device=state.device)
    sink_p = ctypes.c_void_p(sink.data_ptr())
    nbytes = n_maps * 2016 * 4
    calls = {"rmw": (lambda: lib.pcc_probe_rmw(ptr, n_maps, 1.0, 0.0, st), 2 * nbytes),
             "read": (lambda: lib.pcc_probe_read(ptr, n_maps, float("nan"), sink_p, st), nbytes),
             "write": (lambda: lib.pcc_probe_write(ptr, n_maps, 0.5, st), nbytes)}
    out = {}
    for name, (fn, moved) in calls.items():
        if fn() != 0:
            raise RuntimeError(f"probe {name} failed to launch")
        per = 1 if nbytes >= 1 << 30 else 20
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(per):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3 / per)
        out[name + "_gbs"] = moved / float(np.median(times)) / 1e9
    return out


def ceilings(args, wl):
    """The probes and the x_T fill (pc_init_state: write-only, non-temporal) on the workload's state."""
    import numpy as np
    import torch

    import tiled_genome_diffusion_amd as pc

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lay = pc.PCLayout(wl.n_regions, wl.n_guidance, wl.n_traj, wl.chain_len, wl.overlap if wl.chain_len > 1 else 0)
    state = torch.empty(lay.n_maps * pc.PACKED, dtype=torch.float32, device=dev)
    runs = []
    for _ in range(max(1, args.steps)):
        pc.pc_init_state(state, lay, args.seed)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pc.pc_init_state(state, lay, args.seed)
        e1.record(stream)
        torch.cuda.synchronize()
        fill_gbs = lay.n_maps * 2016 * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        runs.append(dict(hbm_probes(state, lay.n_maps, stream), fill_gbs=fill_gbs))
    med = {k: float(np.median([r[k] for r in runs])) for k in runs[0]}
    print(json.dumps({"metric": "HBM ceilings, GB/s", "workload": wl.name, "state_bytes": lay.n_maps * 2016 * 4,
                      "median": med, "runs": runs,
                      "note": "rmw: in-place read-modify-write (bytes read + written); read / write: one "
                              "stream; fill: pc_init_state (x_T, written)"}), flush=True)


def seam_report(args, wl, n_steps):
    """Seam discrepancy of a chain workload at every step: the RMS over the shared pairs per
    (seam, weight, trajectory) before the projection (the fused output of the step kernel) and
    after it (pc_seam_discrepancy), summarised as mean, mean square and max, beside the closed
    form of the expected pre-projection mean square (2 sigma_i^2 from the second step on; the
    first step compares independent draws of x_T).  Then the step time with and without the
    fused discrepancy output, HIP events over whole 50-step loops."""
    import numpy as np
    import torch

    import tiled_genome_diffusion_amd as pc
    from workloads import reference_maps

    if wl.chain_len < 2:
        raise SystemExit("--seam-report needs a chain workload")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lay = pc.PCLayout(wl.n_regions, wl.n_guidance, wl.n_traj, wl.chain_len, wl.overlap)
    x0c, x0u = reference_maps(wl, args.seed)
    x0c_d, x0u_d = torch.from_numpy(x0c).to(dev), torch.from_numpy(x0u).to(dev)
    state = torch.empty(lay.n_maps * pc.PACKED, dtype=torch.float32, device=dev)
    n_cols = lay.n_seams * lay.n_guidance * lay.n_traj
    pre = torch.empty(n_cols, dtype=torch.float32, device=dev)
    rms = torch.empty(n_cols, dtype=torch.float32, device=dev)
    summary = torch.empty(2, dtype=torch.float32, device=dev)
    a_t, a_n = pc.pc_ddim_schedule(n_steps)
    rows = []
    pc.pc_init_state(state, lay, args.seed)
    for i in range(n_steps):
        pc.pc_ddim_cfg_step(state, x0c_d, x0u_d, list(wl.w), lay, a_t[i], a_n[i], wl.eta, args.seed, i + 1,
                            project_seams=True, pre_disc=pre)
        pc.pc_seam_discrepancy(state, lay, rms, summary)
        p = pre.cpu().numpy().astype(np.float64)
        q = rms.cpu().numpy().astype(np.float64)
        a, an = a_t[i], a_n[i]
        sig2 = wl.eta ** 2 * (1 - an) / (1 - a) * (1 - a / an)
        expect = 2 * (1 - an - sig2) / (1 - a) + 2 * sig2 if i == 0 else 2 * sig2
        rows.append({"step": i + 1, "pre_mean": float(p.mean()), "pre_mean_square": float((p * p).mean()),
                     "pre_max": float(p.max()), "expected_pre_mean_square": expect,
                     "post_mean": float(summary[0]), "post_max": float(summary[1]), "post_max_host": float(q.max())})

    def loop(disc):
        pc.pc_init_state(state, lay, args.seed)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n_steps):
            pc.pc_ddim_cfg_step(state, x0c_d, x0u_d, list(wl.w), lay, a_t[i], a_n[i], wl.eta, args.seed, i + 1,
                                project_seams=True, pre_disc=pre if disc else None)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n_steps

    for _ in range(args.warmup):
        loop(False)
        loop(True)
    times = {False: [], True: []}
    for _ in range(max(1, args.steps)):   # interleaved, so clock drift hits both alike
        times[False].append(loop(False))
        times[True].append(loop(True))
    print(json.dumps({"metric": "seam discrepancy before / after projection", "workload": wl.name,
                      "ddim_steps": n_steps, "eta": wl.eta, "seams": lay.n_seams,
                      "joint_samples": lay.n_guidance * lay.n_traj, "pairs_per_seam": wl.overlap * (wl.overlap - 1) // 2,
                      "rows": rows,
                      "step_us_projecting": float(np.median(times[False])),
                      "step_us_projecting_with_discrepancy": float(np.median(times[True]))}), flush=True)


def sync_ablation(args, wl, n_steps):
    """Projection every K steps (ParaChromo's synchronisation interval, section 5.7): wall time of
    the step loop relative to no projection, the paper-form seam discrepancy after the last step and
    averaged over all steps, and the drift of non-overlap entries from the unsynchronised run."""
    import numpy as np
    import torch

    import tiled_genome_diffusion_amd as pc
    from workloads import reference_maps

    if wl.chain_len < 2:
        raise SystemExit("--sync-ablation needs a chain workload")
    dev = torch.device("cuda:0")
    lay = pc.PCLayout(wl.n_regions, wl.n_guidance, wl.n_traj, wl.chain_len, wl.overlap)
    x0c, x0u = reference_maps(wl, args.seed)
    x0c_d, x0u_d = torch.from_numpy(x0c).to(dev), torch.from_numpy(x0u).to(dev)
    state = torch.empty(lay.n_maps * pc.PACKED, dtype=torch.float32, device=dev)
    disc = torch.empty(lay.n_seams * lay.n_guidance, dtype=torch.float32, device=dev)
    a_t, a_n = pc.pc_ddim_schedule(n_steps)
    seam_map = pc.pc_seam_index_map(wl.overlap)   # packed index of each shared pair in the left / right tile
    li, ri = seam_map[:, 0], seam_map[:, 1]
    keep = np.ones((wl.chain_len, pc.PACKED), dtype=bool)
    keep[:-1, li] = False
    keep[1:, ri] = False
    tile = (np.arange(lay.n_maps) // (wl.n_guidance * wl.n_traj)) % wl.chain_len
    keep_d = torch.as_tensor(keep[tile], device=dev)
    mid = n_steps // 2

    def run(K, measure):
        pc.pc_init_state(state, lay, args.seed)
        traj, mid_state = [], None
        for i in range(n_steps):
            proj = K > 0 and (i + 1) % K == 0
            pc.pc_ddim_cfg_step(state, x0c_d, x0u_d, list(wl.w), lay, a_t[i], a_n[i], wl.eta, args.seed, i + 1,
                                project_seams=proj)
            if measure:
                pc.pc_seam_mean_abs(state, lay, disc)
                traj.append(float(disc.mean()))
                if i + 1 == mid:
                    mid_state = state.view(lay.n_maps, pc.PACKED)[keep_d].clone()
        return traj, mid_state

    def once(K):
        # the whole chain from the C side (one launch per step, no host work in between)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        pc.pc_init_state(state, lay, args.seed)
        ev[0].record()
        pc.pc_ddim_sample(state, x0c_d, x0u_d, list(wl.w), lay, n_steps, wl.eta, args.seed, project_every=K,
                          init=False)
        ev[1].record()
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) * 1e-3

    ks = [int(k) for k in args.sync_ablation.split(",")]
    # timings interleaved over all intervals (K = 0 included), so clock and thermal drift hit all alike
    samples = {K: [] for K in [0] + ks}
    for K in samples:
        once(K)
    for _ in range(args.steps):
        for K in samples:
            samples[K].append(once(K))
    t_of = {K: float(np.median(v)) for K, v in samples.items()}
    base_traj, base_mid = run(0, True)
    base_t = t_of[0]
    rows = []
    for K in ks:
        traj, mid_state = run(K, True)
        drift = float(torch.linalg.vector_norm(mid_state - base_mid) / torch.linalg.vector_norm(base_mid))
        t = t_of[K]
        rows.append({"K": K, "step_loop_ms": t * 1e3, "wall_ratio": t / base_t,
                     "final_mean_abs_disc": traj[-1], "mean_abs_disc_over_steps": float(np.mean(traj)),
                     "nonoverlap_drift_at_step_%d" % mid: drift})
    print(json.dumps({"metric": "sync-interval ablation", "workload": wl.name, "ddim_steps": n_steps,
                      "eta": wl.eta, "unsynchronised_step_loop_ms": base_t * 1e3,
                      "unsynchronised_mean_abs_disc_over_steps": float(np.mean(base_traj)),
                      "unsynchronised_final_mean_abs_disc": base_traj[-1], "rows": rows,
                      "note": "point-mass stand-in denoiser: every run ends on the reference maps, so final "
                              "discrepancy and drift do not depend on K"}), flush=True)


def mds_inputs(args, wl):
    """pc_mds_recover on inputs of three kinds, each as many maps as the workload holds, laid out
    like its final state ([R][G][S], map (r, g, s) = the reference that weight g lands on): exact
    maps, maps with seeded 1e-3 relative Gaussian noise (torch's generator on the device), and
    equal mixtures of region r's and region r+1's maps.  HIP events around back-to-back launches
    (median of args.steps, after three untimed ones)."""
    import numpy as np
    import torch

    import tiled_genome_diffusion_amd as pc
    from workloads import reference_maps

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    x0c, x0u = reference_maps(wl, args.seed)
    xc, xu = torch.from_numpy(x0c).to(dev), torch.from_numpy(x0u).to(dev)
    w = torch.tensor(list(wl.w), dtype=torch.float32, device=dev)
    per_rg = (xu[:, None, :] + w[None, :, None] * (xc - xu)[:, None, :])  # [R][G][2016], fp32
    exact = per_rg[:, :, None, :].expand(wl.n_regions, wl.n_guidance, wl.n_traj, 2016).reshape(-1, 2016).contiguous()
    gen = torch.Generator(device=dev).manual_seed(args.seed)
    noisy = exact * (1.0 + 1e-3 * torch.randn(exact.shape, generator=gen, device=dev))
    mixed = 0.5 * (exact + torch.roll(exact, shifts=wl.n_guidance * wl.n_traj, dims=0))
    n = exact.shape[0]
    coords = torch.empty(n * 192, dtype=torch.float32, device=dev)
    rows = {}
    for name, maps in (("exact", exact), ("noisy_1e-3", noisy), ("two_map_mixture", mixed)):
        flat = maps.reshape(-1)
        for _ in range(3):
            pc.pc_mds_recover(flat, coords)
        times = []
        for _ in range(max(1, args.steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            pc.pc_mds_recover(flat, coords)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        gbs = MDS_BYTES_PER_MAP * n / (ms * 1e-3) / 1e9
        rows[name] = {"ms": ms, "maps_per_s": n / (ms * 1e-3), "hbm_gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS}
    print(json.dumps({"metric": "MDS by input kind", "workload": wl.name, "maps": n, "rows": rows}), flush=True)


def chain_kernels(args, wl, n_steps):
    """Per-call times of the chain kernels that sit beside the step loop, on the final state
    and MDS coordinates of one projected pass: HIP events around repeated calls on one stream,
    median over args.steps groups of 20 calls."""
    import numpy as np
    import torch

    import tiled_genome_diffusion_amd as pc
    from workloads import reference_maps

    if wl.chain_len < 2:
        raise SystemExit("--chain-kernels needs a chain workload")
    dev = torch.device("cuda:0")
    lay = pc.PCLayout(wl.n_regions, wl.n_guidance, wl.n_traj, wl.chain_len, wl.overlap)
    x0c, x0u = reference_maps(wl, args.seed)
    x0c_d, x0u_d = torch.from_numpy(x0c).to(dev), torch.from_numpy(x0u).to(dev)
    state = torch.empty(lay.n_maps * pc.PACKED, dtype=torch.float32, device=dev)
    pc.pc_ddim_sample(state, x0c_d, x0u_d, list(wl.w), lay, n_steps, wl.eta, args.seed, project_every=1)
    coords = torch.empty(lay.n_maps * 64 * 3, dtype=torch.float32, device=dev)
    pc.pc_mds_recover(state, coords)
    n_chains = wl.n_regions // wl.chain_len
    n_cols = wl.n_guidance * wl.n_traj
    n_beads = (wl.chain_len - 1) * (64 - wl.overlap) + 64
    chain = torch.empty(n_chains * n_cols * n_beads * 3, dtype=torch.float32, device=dev)
    resid = torch.empty(lay.n_seams * n_cols, dtype=torch.float32, device=dev)
    resid_p = torch.empty_like(resid)
    rms = torch.empty(lay.n_seams * n_cols, dtype=torch.float32, device=dev)
    summary = torch.empty(2, dtype=torch.float32, device=dev)
    mean_abs = torch.empty(lay.n_seams * wl.n_guidance, dtype=torch.float32, device=dev)
    calls = {
        "pc_kabsch_stitch": lambda: pc.pc_kabsch_stitch(coords, lay, chain, resid),
        "pc_kabsch_stitch_proper": lambda: pc.pc_kabsch_stitch_proper(coords, lay, chain, resid_p),
        "pc_seam_mean_abs": lambda: pc.pc_seam_mean_abs(state, lay, mean_abs),
        "pc_seam_discrepancy": lambda: pc.pc_seam_discrepancy(state, lay, rms, summary),
        "pc_seam_project": lambda: pc.pc_seam_project(state, lay),
    }
    rows = {}
    for name, fn in calls.items():
        for _ in range(3):
            fn()
        times = []
        for _ in range(max(1, args.steps)):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(20):
                fn()
            ev[1].record()
            torch.cuda.synchronize()
            times.append(ev[0].elapsed_time(ev[1]) * 1e3 / 20)
        rows[name] = float(np.median(times))
    print(json.dumps({"metric": "chain kernels, microseconds per call", "workload": wl.name,
                      "chains": n_chains, "joint_samples_per_chain": n_cols, "chain_beads": n_beads,
                      "us_per_call": rows,
                      "max_seam_residual": float(resid.max()),
                      "rotations_only": {"max_seam_residual": float(resid_p.max()),
                                         "mirrored_seams": int((resid_p > 1e-2).sum())},
                      "post_projection_rms_max": float(summary[1])}),
          flush=True)


def _oracle_block(name, n_steps, seed, lo, n):
    """The oracle on one block of a workload, one BLAS thread: maps lo .. lo+n-1 of an
    independent workload, or joint-sample columns lo .. lo+n-1 (column c = weight
    c // S, trajectory c % S, every tile) of a chain.  Returns (maps, sampling s, MDS s)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import mds, sampler
    from workloads import get, reference_maps

    wl = get(name)
    G, S = wl.n_guidance, wl.n_traj
    with threadpool_limits(limits=1):
        if wl.chain_len == 1:
            idx = np.arange(lo, lo + n)
            r = idx // (G * S)
            regions = sorted(set(r.tolist()))
            x0c, x0u = reference_maps(wl, seed, regions=regions)
            pos = {v: k for k, v in enumerate(regions)}
            rr = np.array([pos[v] for v in r])
            w = np.asarray(wl.w)[(idx // S) % G]
            t0 = time.perf_counter()
            fin, _ = sampler.run_independent(x0c[rr], x0u[rr], w, idx, seed, n_steps, wl.eta)
            t1 = time.perf_counter()
        else:
            x0c, x0u = reference_maps(wl, seed)
            L = wl.chain_len
            cols = np.arange(lo, lo + n)
            tids = np.array([[(k * G + c // S) * S + c % S for c in cols] for k in range(L)])
            w = np.asarray(wl.w)[cols // S]
            t0 = time.perf_counter()
            fin, _, _, _ = sampler.run_chain(x0c[:L], x0u[:L], w, tids, seed, n_steps, wl.eta, wl.overlap)
            t1 = time.perf_counter()
            fin = fin.reshape(-1, 2016)
        for m in fin:
            mds.classical_mds(m)
        t2 = time.perf_counter()
    return fin.shape[0], t1 - t0, t2 - t1


def _oracle_block_star(args):
    return _oracle_block(*args)


def jacobi_mds_rate(wl, seed, n_maps):
    """maps/s of the oracle's cyclic-Jacobi MDS (the brute-force eigensolver, one thread) on the
    first n_maps reference maps of the workload (final states of the point-mass chain)."""
    from threadpoolctl import threadpool_limits

    from oracle import mds
    from workloads import reference_maps

    if n_maps <= 0:
        return None
    regions = list(range(min(wl.n_regions, (n_maps + 1) // 2))) if wl.chain_len == 1 else None
    x0c, x0u = reference_maps(wl, seed, regions=regions)
    maps = [m for pair in zip(x0c, x0u) for m in pair][:n_maps]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for m in maps:
            mds.classical_mds(m, solver="jacobi")
        dt = time.perf_counter() - t0
    return {"maps": len(maps), "seconds": dt, "maps_per_s": len(maps) / dt}


def cpu_baseline(wl, n_steps, seed, target_s, jacobi_maps=0):
    """Time the oracle (as it stands) on a bounded sample of the workload, one thread."""
    L = wl.chain_len
    n = 16
    n_maps, ts, tm = _oracle_block(wl.name, n_steps, seed, 0, n if L == 1 else max(1, n // L))
    while ts + tm < target_s / 4 and n < wl.n_maps:
        n = min(wl.n_maps, n * 4)
        n_maps, ts, tm = _oracle_block(wl.name, n_steps, seed, 0, n if L == 1 else max(1, n // L))
    return {"value": n_maps * n_steps / (ts + tm), "unit": "trajectory-steps/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_maps} of {wl.n_maps} maps ({wl.name}), {n_steps} float64 DDIM steps + LAPACK MDS, "
                      f"one thread; {ts:.1f} s sampling + {tm:.1f} s MDS",
            "mds_maps_per_s": n_maps / tm, "step_traj_steps_per_s": n_maps * n_steps / ts,
            "jacobi_mds": jacobi_mds_rate(wl, seed, jacobi_maps),
            "host_cpu_count": os.cpu_count(), "host_affinity": len(os.sched_getaffinity(0)),
            "host_cpu_model": cpu_model(), "sample_maps": n_maps}


def cpu_baseline_parallel(wl, n_steps, seed, per_worker_maps, procs):
    """The same oracle in `procs` processes (one BLAS thread each) over disjoint blocks of
    the workload, per_worker_maps maps per process where the workload holds that many:
    the best figure the host's cores reach without changing the oracle."""
    import multiprocessing as mp

    L = wl.chain_len
    units = wl.n_maps if L == 1 else wl.n_guidance * wl.n_traj    # maps, or joint-sample columns
    per = per_worker_maps if L == 1 else max(1, per_worker_maps // L)
    total = min(units, per * procs)
    bounds = [total * j // procs for j in range(procs + 1)]
    blocks = [(wl.name, n_steps, seed, bounds[j], bounds[j + 1] - bounds[j])
              for j in range(procs) if bounds[j + 1] > bounds[j]]
    with mp.get_context("fork").Pool(len(blocks)) as pool:
        t0 = time.perf_counter()
        res = pool.map(_oracle_block_star, blocks, chunksize=1)
        wall = time.perf_counter() - t0
    maps = sum(r[0] for r in res)
    return {"value": maps * n_steps / wall, "unit": "trajectory-steps/s", "cores": len(blocks),
            "kind": "oracle, one process per core",
            "sample": f"{maps} of {wl.n_maps} maps ({wl.name}) in {len(blocks)} blocks, {n_steps} float64 DDIM "
                      f"steps + LAPACK MDS; {wall:.1f} s wall"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the workloads need no inter-GPU communication and the library "
              "runs on a single MI355X; --gpus N > 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import tiled_genome_diffusion_amd as pc
    from workloads import get, reference_maps

    wl = get(args.workload)
    if args.warmup is None:
        args.warmup = 1 if wl.n_maps * 2016 * 4 >= 1 << 30 else 30
    if args.traffic_summary:
        return traffic_summary(args, wl)
    if args.copy_only:
        return copy_only(args, wl)
    n_steps = args.n_steps or wl.n_steps[0]
    if args.cpu_only:
        out = {"workload": wl.name, "ddim_steps": n_steps,
               "cpu_baseline": cpu_baseline(wl, n_steps, args.seed, args.cpu_seconds, args.jacobi_maps)}
        if args.cpu_procs > 0:
            out["cpu_baseline_parallel"] = cpu_baseline_parallel(
                wl, n_steps, args.seed, out["cpu_baseline"]["sample_maps"], args.cpu_procs)
        print(json.dumps(out), flush=True)
        return None
    if args.sync_ablation:
        return sync_ablation(args, wl, n_steps)
    if args.chain_kernels:
        return chain_kernels(args, wl, n_steps)
    if args.ceilings:
        return ceilings(args, wl)
    if args.seam_report:
        return seam_report(args, wl, n_steps)
    if args.mds_inputs:
        return mds_inputs(args, wl)
    dev = torch.device("cuda:0")
    lay = pc.PCLayout(wl.n_regions, wl.n_guidance, wl.n_traj, wl.chain_len, wl.overlap if wl.chain_len > 1 else 0)
    seeds = [int(v) for v in args.seeds.split(",")]
    if args.graph:
        seeds = seeds[:1]   # a captured graph holds one seed
    refs = {}
    for sd in seeds:
        x0c, x0u = reference_maps(wl, sd)
        refs[sd] = (torch.from_numpy(x0c).to(dev), torch.from_numpy(x0u).to(dev))
    state = torch.empty(lay.n_maps * pc.PACKED, dtype=torch.float32, device=dev)
    coords = torch.empty(lay.n_maps * 64 * 3, dtype=torch.float32, device=dev)
    project = 1 if wl.chain_len > 1 else 0
    stream = torch.cuda.current_stream(dev)
    if args.eps_buffers:
        # stand-ins for a network's per-map outputs, drawn once; each step reads both
        gen = torch.Generator(device=dev).manual_seed(seeds[0])
        eps_c = torch.randn(lay.n_maps * pc.PACKED, generator=gen, device=dev)
        eps_u = torch.randn(lay.n_maps * pc.PACKED, generator=gen, device=dev)
        a_t, a_n = pc.pc_ddim_schedule(n_steps)

    def one_pass(events=None, sd=seeds[0]):
        if events:
            events[3].record(stream)
        if args.eps_buffers:
            pc.pc_init_state(state, lay, sd)
            if events:
                events[0].record(stream)
            for i in range(n_steps):
                pc.pc_ddim_cfg_step_eps(state, eps_c, eps_u, list(wl.w), lay, a_t[i], a_n[i], wl.eta, sd,
                                        i + 1, project_seams=bool(project))
        else:
            if events:
                events[0].record(stream)
            # x_T is drawn inside the first step (no fill, no read of the state)
            pc.pc_ddim_sample(state, refs[sd][0], refs[sd][1], list(wl.w), lay, n_steps, wl.eta, sd,
                              project_every=project, init=True)
        if events:
            events[1].record(stream)
        pc.pc_mds_recover(state, coords)
        if events:
            events[2].record(stream)

    for k in range(args.warmup):
        one_pass(sd=seeds[k % len(seeds)])
    torch.cuda.synchronize()

    # events per pass: [3] pass start, [0] step loop start (after the fill in the eps-buffer form;
    # otherwise x_T is drawn by the first step), [1] after the step loop, [2] after MDS
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    if args.graph:
        # three graphs per pass (x_T, the step loop, MDS); the events go between the replays
        sd0 = seeds[0]

        def seg_init():
            pc.pc_init_state(state, lay, sd0)

        def seg_steps():
            if args.eps_buffers:
                for i in range(n_steps):
                    pc.pc_ddim_cfg_step_eps(state, eps_c, eps_u, list(wl.w), lay, a_t[i], a_n[i], wl.eta,
                                            sd0, i + 1, project_seams=bool(project))
            else:
                pc.pc_ddim_sample(state, refs[sd0][0], refs[sd0][1], list(wl.w), lay, n_steps, wl.eta, sd0,
                                  project_every=project, init=True)

        def seg_mds():
            pc.pc_mds_recover(state, coords)

        graphs = []
        for seg in ((seg_init,) if args.eps_buffers else ()) + (seg_steps, seg_mds):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                seg()
            graphs.append(g)
        if not args.eps_buffers:
            graphs.insert(0, None)   # x_T is drawn inside the step-loop graph

        def one_pass(events=None, sd=sd0):  # noqa: F811 - the graph-replay form of the pass
            if events:
                events[3].record(stream)
            if graphs[0] is not None:
                graphs[0].replay()
            if events:
                events[0].record(stream)
            graphs[1].replay()
            if events:
                events[1].record(stream)
            graphs[2].replay()
            if events:
                events[2].record(stream)

        one_pass()
        torch.cuda.synchronize()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        one_pass(evs[k], seeds[k % len(seeds)])
    torch.cuda.synchronize()
    t1 = time.perf_counter()

    # per-seed rates from the GPU time of each pass (x_T + steps + MDS)
    traj_steps = lay.n_maps * n_steps
    per_seed = {}
    for k, e in enumerate(evs):
        per_seed.setdefault(seeds[k % len(seeds)], []).append(e[3].elapsed_time(e[2]))
    by_seed = {str(sd): traj_steps / (float(np.mean(v)) * 1e-3) for sd, v in per_seed.items()}

    # the ceiling of the step kernel's access pattern on this device: the in-place read-modify-write
    # probe over the same state (which it overwrites; the passes are done with it)
    probes = hbm_probes(state, lay.n_maps, stream)

    ms_per_pass = (t1 - t0) * 1e3 / args.steps
    step_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    mds_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    launch_ms = step_ms / n_steps
    if args.eps_buffers:
        bytes_per_launch = lay.n_maps * STEP_BYTES_PER_MAP * 2   # + both noise predictions read
        loop_bytes = n_steps * bytes_per_launch
    else:
        bytes_per_launch = lay.n_maps * STEP_BYTES_PER_MAP + lay.n_regions * REF_BYTES_PER_REGION
        # the first step draws x_T instead of reading it: it only writes the state
        loop_bytes = n_steps * bytes_per_launch - lay.n_maps * STEP_BYTES_PER_MAP // 2
    achieved = loop_bytes / (step_ms * 1e-3) / 1e9
    traffic, traffic_kernel = measured_traffic(wl.name) if not args.eps_buffers else (None, None)

    out = {
        "metric": "DDIM trajectory-steps/s (64-bead maps) + % HBM peak; MDS maps/s",
        "value": traj_steps / (ms_per_pass * 1e-3),
        "unit": "trajectory-steps/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_pass,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "maps": lay.n_maps, "regions": wl.n_regions, "guidance": wl.n_guidance,
                   "trajectories": wl.n_traj, "chain_len": wl.chain_len, "ddim_steps": n_steps, "eta": wl.eta,
                   "seeds": seeds, "denoiser": "noise-prediction buffers" if args.eps_buffers else "point-mass",
                   "launch": "HIP graph replay" if args.graph else "eager",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "k_step_indep" if wl.chain_len == 1 else "k_step_chain",
                     "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-scaled)",
                     "traffic_kernel": traffic_kernel, "launch_us": launch_ms * 1e3,
                     # achieved = bytes_per_launch / launch_us: both averaged over the loop's launches
                     "bytes_per_launch": loop_bytes / n_steps, "step_loop_bytes": loop_bytes,
                     # a launch that reads and writes the whole state: the basis of `traffic`
                     "bytes_per_steady_launch": bytes_per_launch,
                     # measured live: the step's state access pattern with one FMA per element
                     "ceiling": probes["rmw_gbs"], "frac_of_ceiling": achieved / probes["rmw_gbs"],
                     "ceiling_kind": "in-place float4 read-modify-write probe, step kernel's mapping and cache policy",
                     "read_ceiling": probes["read_gbs"], "write_ceiling": probes["write_gbs"]},
        "value_by_seed": by_seed,
        "value_sd_over_seeds": float(np.std(list(by_seed.values()), ddof=1)) if len(by_seed) > 1 else None,
        "step_loop_traj_steps_per_s": traj_steps / (step_ms * 1e-3),
        "mds_maps_per_s": lay.n_maps / (mds_ms * 1e-3),
        "mds_ms": mds_ms,
        # MDS moves 8,832 B and does about 90.6 k flops per map (10.3 flop/B).  Against 8 TB/s the bytes
        # take 1.10 ns per map, the flops 1.15 ns at the non-packed FP32 peak (0.58 ns at the packed
        # peak and on the matrix cores, which run two thirds of them): the two bounds meet, and the
        # line reports the HBM one with the flop rate beside it
        "mds_roofline": {"bound": "hbm", "kernel": "k_mds", "unit": "GB/s", "peak": HBM_PEAK_GBS,
                         "achieved": MDS_BYTES_PER_MAP * lay.n_maps / (mds_ms * 1e-3) / 1e9,
                         "frac": MDS_BYTES_PER_MAP * lay.n_maps / (mds_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "bytes_per_map": MDS_BYTES_PER_MAP, "flops_per_map": MDS_FLOPS_PER_MAP,
                         "tflops": MDS_FLOPS_PER_MAP * lay.n_maps / (mds_ms * 1e-3) / 1e12,
                         "frac_of_nonpacked_fp32": MDS_FLOPS_PER_MAP * lay.n_maps / (mds_ms * 1e-3) / 1e12
                         / FP32_NONPACKED_PEAK_TFLOPS,
                         "nonpacked_fp32_peak": FP32_NONPACKED_PEAK_TFLOPS,
                         "published_fp32_peak_counting_packed": FP32_PEAK_TFLOPS},
        "step_loop_ms": step_ms,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, n_steps, args.seed, args.cpu_seconds, args.jacobi_maps)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
