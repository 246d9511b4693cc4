#!/usr/bin/env python3
"""Benchmark of the Lloyd k-means hot path on one MI355X.

A step is one Lloyd iteration (``kmeans_lloyd_step``: centroid norms, sample
norms, fused MFMA assignment with the argmin in the register epilogue,
finalize, counts, stable grouping by label, segmented float64 sums and the
mean) over the whole workload, inputs resident in HBM. Default workload: the
feature-heavy shape, n = 65536 samples, k = 4096 centroids, d = 16384 features,
float32, seeded synthetic Gaussian blobs.

Prints one JSON line:
  value        2*n*k*d / (Lloyd step time), TFLOP/s (whole step, update included)
  ms_per_step  Lloyd iteration time in ms
  assign_*     the fused assignment alone (kmeans_assign without min_dist)
  update_*     the centroid update alone (kmeans_update) and its HBM rate
  roofline     the fused assignment kernel against the MI355X fp32 MFMA peak
  cpu_baseline the float64 oracle on a bounded sample of rows, host cores
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC_FMT = "fused assign TFLOP/s (2nkd/t) + Lloyd iteration ms, {n}×{k}×{d} fp32"
# The headline line: the feature-heavy workload.
METRIC = METRIC_FMT.format(n=65536, k=4096, d=16384)
MFMA_FP32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix peak (published)
HBM_PEAK_GBPS = 8000.0         # MI355X HBM3E bandwidth (published)
# The pages' k-means++ time on an NVIDIA L4 at 65536 x 1024 x 8192 (context).
PAGES_KMEANSPP_MS = 10300.0
# The pages' Lloyd-iteration times on an NVIDIA L4, per workload (context).
PAGES_LLOYD_MS = {"feature_heavy": 1700.0, "centroid_heavy": 3853.0}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "assign_dma_feature_heavy_traffic.json")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def prewarm(step, ms: float) -> int:
    """Run `step` untimed until at least `ms` of wall time has passed (at
    least once); returns the number of runs."""
    import torch

    runs = 0
    t0 = time.perf_counter()
    while True:
        step()
        runs += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return runs


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="before the warmup steps, run the step untimed for at least this "
                         "long: the GPU's clocks ramp up over the first tens of ms of "
                         "sustained work (a short kernel runs ~15 %% slower until then)")
    ap.add_argument("--config", default="feature_heavy",
                    help="workload name (tiny, probe, mid, sample_heavy, feature_heavy, "
                         "centroid_heavy)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target duration of the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["lloyd", "fit", "kmeanspp"], default="lloyd",
                    help="lloyd: one Lloyd step per timed step (default); fit: kmeans_fit "
                         "with relocation running exactly --steps iterations; kmeanspp: greedy "
                         "k-means++ seeding of k centres (use --config kmeanspp for the pages' "
                         "65536 x 1024 x 8192 shape)")
    return ap.parse_args()


def assign_kernel_name(n: int, k: int, d: int, cus: int = 256) -> str:
    """The product kernel kmeans_assign runs for 16-byte aligned inputs of
    this shape on a device with `cus` compute units (the launcher's rule: the
    small-k kernel with C resident in LDS for k <= 64, or k <= 128 from 2^17
    samples, where C fits in 64 KiB;
    else DMA-staged 256 x 256 tiles when d is a multiple of 4, there are at least
    256 of them and either every tile is full (d a multiple of 64) or 1.8
    rounds of 128 x 256 tiles per round of them still come out ahead)."""
    def cdiv(a, b):
        return -(-a // b)

    # Small k (up to 64, or 128 from 2^17 samples): C resident in LDS
    # (16-row blocks, rows of d rounded up to 64 plus 4 floats, at most 64 KiB).
    small = k <= 64 or (k <= 128 and n >= 1 << 17)
    if small and d % 4 == 0 and 16 * cdiv(k, 16) * (cdiv(d, 64) * 64 + 4) <= 16384:
        return "assign_smallk_kernel"

    def rounds(tiles):
        return cdiv(cdiv(tiles, 8), max(cus // 8, 1))

    big = cdiv(n, 256) * cdiv(k, 256)
    mid = cdiv(n, 256) * cdiv(k, 128)
    if d % 4 == 0 and big >= 256:
        if n % 256 == 0 and k % 256 == 0 and d % 64 == 0:
            return "assign_dma_kernel"
        if mid >= 512 and 9 * rounds(big) < 5 * rounds(mid):
            return "assign_dma_kernel"
    return "assign_tile_kernel"


def traffic_record(cfg):
    """Bytes per launch of the assignment kernel beyond its L2 from committed
    rocprofv3 counter runs (FETCH_SIZE + WRITE_SIZE, each scaled by the factor
    a plain copy kernel of known size gives; FETCH_SIZE includes what the
    MALL in front of HBM serves, so this bounds the HBM bytes from above), or
    None when absent or when the kernel source has changed since the counters
    were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    from nearest_centroid_assignment_amd.profile_run import kernel_digest

    if rec.get("assign_kernel_sha256") != kernel_digest() or rec.get("workload") != cfg.name:
        return None
    return rec.get("beyond_l2_bytes_per_launch")


def host_info() -> dict:
    """What the CPU baseline ran on: the CPU model, the CPUs this process may
    use and OMP_NUM_THREADS as set (None when unset)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        cpus = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        cpus = os.cpu_count()
    return {"cpu_model": model, "cpus_available": cpus,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(X, C, target_s: float):
    """Time the float64 oracle's assignment on a seeded sample of rows against
    all centroids; scale to TFLOP/s of the same 2*rows*k*d work. The sample
    grows until one timed batch takes at least half of ``target_s``."""
    import numpy as np

    import oracle

    k, d = C.shape
    rng = np.random.default_rng(7)
    order = rng.permutation(len(X))
    m = min(len(X), 64)
    while True:
        Xs = np.ascontiguousarray(X[np.sort(order[:m])])
        t0 = time.perf_counter()
        oracle.assign(Xs, C)
        t = time.perf_counter() - t0
        if t >= 0.5 * target_s or m == len(X):
            break
        m = int(min(len(X), max(2 * m, m * target_s / max(t, 1e-3))))
    return {
        "value": 2.0 * m * k * d / t / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{m} seeded rows x all {k} centroids x {d} features "
                  f"(float64 difference-form assignment, {t:.1f} s)",
        **host_info(),
    }


def cpu_baseline_kmeanspp(X, k, first, trials, rand, target_s: float):
    """Time the float64 oracle's seeding of the first m centres (same draws),
    m growing until one run takes at least half of ``target_s``; every centre
    after the first costs the same, so the full seeding is estimated as
    t(m) * (k - 1) / (m - 1) ms."""
    import oracle

    m = min(k, 3)
    while True:
        t0 = time.perf_counter()
        oracle.kmeanspp(X, m, first, trials, rand[: m - 1])
        t = time.perf_counter() - t0
        if t >= 0.5 * target_s or m == k:
            break
        m = int(min(k, max(m + 1, 1 + (m - 1) * target_s / max(t, 1e-3))))
    scale = (k - 1) / (m - 1) if m > 1 else 1.0
    return {
        "value": round(t * 1e3 * scale, 1),
        "unit": "ms",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"first {m} of {k} centres of the same seeding (float64 difference form, "
                  f"{t:.1f} s), scaled by (k - 1) / (m - 1)",
        **host_info(),
    }


def bench_fit(args, cfg, Xg, Cg, labels, md, counts, stream) -> int:
    """kmeans_fit with empty-cluster relocation, forced to run exactly
    --steps iterations (tol = -1), against --steps separate Lloyd steps."""
    import torch

    from nearest_centroid_assignment_amd import binding

    n, k, d = cfg.n, cfg.k, cfg.d
    dev = Xg.device
    C_out = torch.empty_like(Cg)
    info = torch.empty(3, dtype=torch.float64, device=dev)
    wsb = binding.kmeans_workspace_bytes(n, k, d, binding.KM_OP_FIT)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)

    def fit(iters):
        binding.kmeans_fit(Xg, Cg, iters, -1.0, binding.KM_FIT_RELOCATE_EMPTY, C_out, labels,
                           md, counts, info, workspace=ws, stream=stream)

    pre = prewarm(lambda: fit(1), args.prewarm_ms)
    log(f"prewarm: {pre} one-iteration fits; fit warmup ({args.warmup} iterations)")
    fit(max(1, args.warmup))
    torch.cuda.synchronize()
    log(f"timing fit with {args.steps} iterations")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    fit(args.steps)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3
    total_ms = ev0.elapsed_time(ev1)
    n_iter = int(info[0].item())
    # The call ends with one more assignment against the final centres; time
    # that assignment alone to report the cost of an iteration without it.
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    binding.kmeans_assign(Xg, C_out, labels, md, stream=stream)
    a1.record(stream)
    torch.cuda.synchronize()
    final_assign_ms = a0.elapsed_time(a1)
    per_iter = (total_ms - final_assign_ms) / max(n_iter, 1)
    result = {
        "metric": "kmeans_fit ms (iterations of assignment + relocation + update + convergence "
                  "check, then a final assignment)",
        "value": round(total_ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_steps": pre,
        "ms_per_step": round(per_iter, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} n={n} k={k} d={d} float32 Gaussian blobs, seed 0",
                   "n": n, "k": k, "d": d, "iterations": n_iter},
        "fit_wall_ms": round(wall_ms, 3),
        "final_assign_ms": round(final_assign_ms, 3),
        "ms_per_iteration": round(per_iter, 3),
        "inertia": info[1].item(),
        "tflops_per_iter": round(cfg.flops / (per_iter * 1e-3) / 1e12, 3),
        "workspace_bytes": wsb,
    }
    print(json.dumps(result), flush=True)
    return 0


def bench_kmeanspp(args, cfg, X, Xg, stream) -> int:
    """Greedy k-means++ seeding of cfg.k centres (2 + log(k) trials) with
    seeded draws; --steps timed runs after --warmup."""
    import torch

    import oracle
    from nearest_centroid_assignment_amd import binding, datagen

    n, k, d = cfg.n, cfg.k, cfg.d
    trials = oracle.default_trials(k)
    first, rand = datagen.make_seeding_draws(n, k, trials)
    rg = torch.from_numpy(rand.reshape(-1).copy()).to(Xg.device)
    centres = torch.empty((k, d), dtype=torch.float32, device=Xg.device)
    chosen = torch.empty(k, dtype=torch.int64, device=Xg.device)
    wsb = binding.kmeans_workspace_bytes(n, k, d, binding.KM_OP_KMEANSPP)
    ws = torch.empty(wsb, dtype=torch.uint8, device=Xg.device)

    def run():
        binding.kmeans_plusplus(Xg, k, first, trials, rg, centres, chosen, workspace=ws,
                                stream=stream)

    pre = prewarm(run, args.prewarm_ms)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    times = []
    for _ in range(args.steps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    ms = sorted(times)[len(times) // 2]
    # Bytes the distance kernels must read: X once per centre.
    x_bytes = 4.0 * n * d * k
    # Algorithmic bytes of the distance launches: per launch X (4nd), the
    # previous D (8n), the new D of every trial (8n per trial) and the
    # candidate rows (4d per trial); the first launch has one trial and no
    # previous D. Attributed to the whole seeding time (which also holds the
    # selection launches and the sample norms), so this underestimates the
    # distance kernel's own rate.
    dist_bytes = (4.0 * n * d + 8.0 * n + 4.0 * d) + (k - 1) * (
        4.0 * n * d + 8.0 * n + trials * (8.0 * n + 4.0 * d))
    achieved = dist_bytes / (ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None}
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle k-means++ on a prefix of the centres")
        cpu = cpu_baseline_kmeanspp(X, k, first, trials, rand, args.cpu_seconds)
    result = {
        "metric": "k-means++ seeding ms (greedy, 2 + log(k) trials)",
        "value": round(ms, 3),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_steps": pre,
        "ms_per_step": round(ms, 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": (round(PAGES_KMEANSPP_MS / ms, 2)
                        if (n, k, d) == (65536, 1024, 8192) else None),
        "dtype": "f64 distances on f32 samples",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} n={n} k={k} d={d} float32 Gaussian blobs, seed 0",
                   "n": n, "k": k, "d": d, "trials": trials},
        "x_read_gbps": round(x_bytes / (ms * 1e-3) / 1e9, 1),
        "workspace_bytes": wsb,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)
    return 0


def main() -> int:
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(a sample-sharded run would give each GPU n/G rows and a copy of C, run "
              "the same kernels on its shard and all-reduce the per-cluster sums and "
              "counts).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from nearest_centroid_assignment_amd import binding, datagen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    cfg = datagen.CONFIGS[args.config]
    n, k, d = cfg.n, cfg.k, cfg.d
    dev = torch.device("cuda:0")

    log(f"generating {cfg.name} {n}x{k}x{d}")
    X, C = datagen.make(cfg)
    Xg = torch.from_numpy(X).to(dev)
    Cg = torch.from_numpy(C).to(dev)
    labels = torch.empty(n, dtype=torch.int64, device=dev)
    md = torch.empty(n, dtype=torch.float32, device=dev)
    C_new = torch.empty_like(Cg)
    counts = torch.empty(k, dtype=torch.int64, device=dev)
    ws_bytes = binding.kmeans_workspace_bytes(n, k, d, binding.KM_OP_LLOYD)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()

    def lloyd():
        binding.kmeans_lloyd_step(Xg, Cg, labels, md, C_new, counts, workspace=ws, stream=stream)

    if args.mode == "fit":
        return bench_fit(args, cfg, Xg, Cg, labels, md, counts, stream)
    if args.mode == "kmeanspp":
        return bench_kmeanspp(args, cfg, X, Xg, stream)

    def assign_only():
        binding.kmeans_assign(Xg, Cg, labels, None, workspace=ws, stream=stream)

    pre = prewarm(lloyd, args.prewarm_ms)
    log(f"prewarm {pre} steps, warmup {args.warmup}")
    for _ in range(args.warmup):
        lloyd()
    torch.cuda.synchronize()

    # Timed Lloyd steps: events on the stream the kernels run on, bracketed by
    # device synchronisation; the wall clock is kept beside the events.
    torch.cuda.reset_peak_memory_stats(dev)
    base_alloc = torch.cuda.memory_allocated(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} Lloyd steps")
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        lloyd()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - w0) * 1e3 / args.steps
    lloyd_ms = ev0.elapsed_time(ev1) / args.steps
    peak_extra = torch.cuda.max_memory_allocated(dev) - base_alloc

    # The fused assignment alone, one event pair per call, for the roofline of
    # its dominant kernel (the three tiny kernels around it are included, so
    # the kernel's own rate is slightly higher than reported).
    # Launch-bound shapes (tiny, probe) take at least 50 calls.
    areps = args.steps if cfg.flops >= 1e10 else max(args.steps, 50)
    log(f"timing {areps} assignments")
    assign_only()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(areps)]
    for a, b in evs:
        a.record(stream)
        assign_only()
        b.record(stream)
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) for a, b in evs)
    assign_ms = sum(per_call) / len(per_call)
    flops = cfg.flops
    assign_tflops = flops / (assign_ms * 1e-3) / 1e12

    # The update alone (labels from the assignments just timed), for its HBM
    # rate: algorithmic bytes = X once (4nd), the labels once (8n) and the new
    # centres (4kd). The updates run back to back between one event pair, like
    # the Lloyd steps; one assignment is enqueued first, so that the host has
    # queued them before the GPU gets there (an update of 0.1 ms is otherwise
    # timed partly as the host's time to launch it).
    log(f"timing {args.steps} updates")
    u0, u1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    assign_only()
    u0.record(stream)
    for _ in range(args.steps):
        binding.kmeans_update(Xg, labels, Cg, C_new, counts, workspace=ws, stream=stream)
    u1.record(stream)
    torch.cuda.synchronize()
    update_ms = u0.elapsed_time(u1) / args.steps
    update_gbps = (4.0 * n * d + 8.0 * n + 4.0 * k * d) / (update_ms * 1e-3) / 1e9

    traffic = traffic_record(cfg)
    roofline = {
        "bound": "mfma",
        "achieved": round(assign_tflops, 3),
        "peak": MFMA_FP32_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(assign_tflops / MFMA_FP32_PEAK_TFLOPS, 4),
        "traffic": traffic,
        "kernel": assign_kernel_name(n, k, d, torch.cuda.get_device_properties(0).multi_processor_count),
        "algorithmic_per_launch": f"2*n*k*d = {flops:.4e} flop",
    }

    result = {
        "metric": METRIC_FMT.format(n=cfg.n, k=cfg.k, d=cfg.d),
        "value": round(flops / (lloyd_ms * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm_steps": pre,
        "ms_per_step": round(lloyd_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(PAGES_LLOYD_MS[cfg.name] / lloyd_ms, 2)
                        if cfg.name in PAGES_LLOYD_MS else None),
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name} n={n} k={k} d={d} float32 Gaussian blobs, seed 0",
                   "n": n, "k": k, "d": d},
        "lloyd_ms": round(lloyd_ms, 3),
        "lloyd_wall_ms": round(wall_ms, 3),
        "assign_ms": round(assign_ms, 3),
        "assign_ms_min": round(per_call[0], 3),
        "assign_ms_median": round(per_call[len(per_call) // 2], 3),
        "assign_calls": len(per_call),
        "assign_tflops": round(assign_tflops, 3),
        "update_ms": round(update_ms, 3),
        "update_hbm_gbps": round(update_gbps, 1),
        "update_frac_of_hbm_peak": round(update_gbps / HBM_PEAK_GBPS, 4),
        "workspace_bytes": ws_bytes,
        # labels 8n + min_dist 4n + C_new 4kd + counts 8k, allocated by the caller
        "outputs_bytes": 12 * n + 4 * k * d + 8 * k,
        "workspace_plus_outputs_bytes": ws_bytes + 12 * n + 4 * k * d + 8 * k,
        "peak_extra_bytes_during_step": int(peak_extra),
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        log("timing the oracle CPU baseline")
        result["cpu_baseline"] = cpu_baseline(X, C, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
