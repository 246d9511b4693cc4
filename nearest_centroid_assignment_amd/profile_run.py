"""Driver and summarizer for the rocprofv3 hardware-counter runs.

run (default):
    python3 -m nearest_centroid_assignment_amd.profile_run [--workload feature_heavy]
        [--op assign|update|kmeanspp]
  launches, in order and each once: a 1 GiB streaming copy (calibration), then
  on the workload's seeded inputs either one ``kmeans_assign`` (no min_dist;
  op assign) or one ``kmeans_assign`` followed by one ``kmeans_update`` with
  its labels (op update), or one k-means++ seeding of k centres (op kmeanspp).
  Meant to be run under ``rocprofv3 --pmc FETCH_SIZE``
  and, separately, under ``rocprofv3 --pmc WRITE_SIZE`` (csv output), or with
  other counters.

summarize:
    python3 -m nearest_centroid_assignment_amd.profile_run summarize \
        --fetch <dir of the FETCH_SIZE run> --write <dir of the WRITE_SIZE run> \
        --out profiles/assign_tile_feature_heavy_traffic.json
  reads the counter_collection csv files, scales each counter of the
  assignment kernel by (known copy bytes / what the same counter read for the
  copy kernel), and records the bytes per launch together with a SHA-256 of
  csrc/assign.hip and its compile flags, so that a later change to the kernel
  voids it. FETCH_SIZE counts what the L2 fetches from beyond itself (HBM and
  the MALL in front of it), so the figure is beyond-L2 traffic, an upper
  bound of the HBM bytes.

trace:
    python3 -m nearest_centroid_assignment_amd.profile_run trace \
        --dir <run dir> --workload mid --bench-line <file> --out <file.md>
  writes the kernel-trace summary of a run of
  ``rocprofv3 --kernel-trace --stats --output-format csv -d <run dir> -o bench
  -- python3 -u bench.py --config <workload> --steps 5 --warmup 1
  --no-cpu-baseline`` (its stdout, the bench line, saved in <file>): every
  kernel's calls, average and minimum duration and share of the time, the
  assignment's product kernel as a fraction of the fp32 MFMA peak (over all
  its calls and over the timed assignment calls alone, the last ones before
  the final assignment), the plain update's mean kernel in bytes per second,
  and bench.py's own figures.

kernels:
    python3 -m nearest_centroid_assignment_amd.profile_run kernels \
        --dir <run dir> [--dir <run dir> ...]
  prints, for every kernel in the runs' counter_collection csv files, each
  counter's average per dispatch; FETCH_SIZE and WRITE_SIZE are also given in
  bytes, scaled by what the counter read for the copy kernel.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ASSIGN_SOURCE = os.path.join(HERE, "csrc", "assign.hip")
COPY_BYTES = 1 << 30
COPY_KERNEL = "copy_kernel"
# The assignment's product kernel: the DMA-staged 256 x 256 one on the full
# large shapes, the small-k one for k <= 64, the register-staged one elsewhere.
ASSIGN_KERNELS = ("assign_dma_kernel", "assign_smallk_kernel", "assign_tile_kernel")


def kernel_digest() -> str:
    """SHA-256 of what defines the assignment kernel's code: its source file
    and the hipcc flags it is compiled with."""
    from . import build

    h = hashlib.sha256()
    with open(ASSIGN_SOURCE, "rb") as f:
        h.update(f.read())
    h.update(json.dumps([build.HIPCC_FLAGS, build.EXTRA_FLAGS.get("assign.hip", [])]).encode())
    return h.hexdigest()


def run(workload: str, op: str = "assign") -> None:
    import torch

    from . import binding, calib, datagen

    dev = torch.device("cuda:0")
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    print(f"[profile_run] copy {COPY_BYTES} bytes", flush=True)
    calib.copy_once(dst, src, COPY_BYTES)
    torch.cuda.synchronize()
    del src, dst
    cfg = datagen.CONFIGS[workload]
    X, C = datagen.make(cfg)
    Xg, Cg = torch.from_numpy(X).to(dev), torch.from_numpy(C).to(dev)
    if op == "kmeanspp":
        # The seeding's trial count 2 + floor(ln k) (the pages' 2 + log k), here
        # written out so that this module needs nothing from the oracle.
        import math

        trials = 2 + int(math.log(cfg.k))
        first, rand = datagen.make_seeding_draws(cfg.n, cfg.k, trials)
        rg = torch.from_numpy(rand.reshape(-1).copy()).to(dev)
        torch.cuda.synchronize()
        print(f"[profile_run] kmeans_plusplus {cfg.name} {cfg.n}x{cfg.d}, k={cfg.k}", flush=True)
        binding.plusplus(Xg, cfg.k, first, trials, rg)
        torch.cuda.synchronize()
        print("[profile_run] done", flush=True)
        return
    labels = torch.empty(cfg.n, dtype=torch.int64, device=dev)
    torch.cuda.synchronize()
    print(f"[profile_run] kmeans_assign {cfg.name} {cfg.n}x{cfg.k}x{cfg.d}", flush=True)
    binding.kmeans_assign(Xg, Cg, labels, None)
    torch.cuda.synchronize()
    if op == "update":
        C_new = torch.empty_like(Cg)
        counts = torch.empty(cfg.k, dtype=torch.int64, device=dev)
        print(f"[profile_run] kmeans_update {cfg.name}", flush=True)
        binding.kmeans_update(Xg, labels, Cg, C_new, counts)
        torch.cuda.synchronize()
    print("[profile_run] done", flush=True)


def _counter_rows(run_dir: str, counter: str):
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {run_dir}")
    rows = []
    for f in files:
        with open(f, newline="") as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append(r)
    return rows


def _per_kernel(rows, name_part):
    """Counter values of the dispatches whose kernel name contains name_part
    (a string, or a tuple of alternatives tried in order)."""
    parts = (name_part,) if isinstance(name_part, str) else tuple(name_part)
    for part in parts:
        vals = [float(r["Counter_Value"]) for r in rows if part in r.get("Kernel_Name", "")]
        if vals:
            return vals
    raise ValueError(f"no dispatch of a kernel named *{parts}* in the counter rows")


def _kernel_found(rows, parts) -> str:
    for part in parts:
        if any(part in r.get("Kernel_Name", "") for r in rows):
            return part
    return ""


def summarize(fetch_dir: str, write_dir: str, out: str, workload: str) -> dict:
    from .datagen import CONFIGS

    cfg = CONFIGS[workload]
    rec = {"workload": workload, "copy_bytes": COPY_BYTES}
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        copy_kib = _per_kernel(rows, COPY_KERNEL)[0]
        assign_kib = _per_kernel(rows, ASSIGN_KERNELS)
        rec["assign_kernel"] = _kernel_found(rows, ASSIGN_KERNELS)
        scale = (COPY_BYTES / 1024.0) / copy_kib
        per_launch = sum(assign_kib) / len(assign_kib) * scale * 1024.0
        rec[counter] = {"copy_kib": copy_kib, "assign_kib_per_launch": assign_kib,
                        "scale": scale, "assign_bytes_per_launch": per_launch}
        total += per_launch
    alg = 4.0 * (cfg.n * cfg.d + cfg.k * cfg.d) + 8.0 * cfg.n
    rec["beyond_l2_bytes_per_launch"] = total
    rec["algorithmic_min_bytes"] = alg
    rec["traffic_over_min"] = total / alg
    rec["assign_kernel_sha256"] = kernel_digest()
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


def kernel_table(dirs) -> list:
    """Per kernel (full name) and counter: dispatches and average value; for
    FETCH_SIZE / WRITE_SIZE also bytes per dispatch, scaled by the copy."""
    by = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        for f in files:
            with open(f, newline="") as fh:
                for r in csv.DictReader(fh):
                    key = (r.get("Kernel_Name", ""), r.get("Counter_Name", ""))
                    by.setdefault(key, {}).setdefault(r.get("Dispatch_Id", len(by)), 0.0)
                    by[key][r.get("Dispatch_Id", len(by))] += float(r["Counter_Value"])
    scale = {}
    for (kname, cname), disp in by.items():
        if COPY_KERNEL in kname and cname in ("FETCH_SIZE", "WRITE_SIZE"):
            scale[cname] = (COPY_BYTES / 1024.0) / (sum(disp.values()) / len(disp))
    rows = []
    for (kname, cname), disp in sorted(by.items()):
        avg = sum(disp.values()) / len(disp)
        row = {"kernel": kname, "counter": cname, "dispatches": len(disp), "average": avg}
        if cname in scale:
            row["bytes"] = avg * scale[cname] * 1024.0
            row["scale"] = scale[cname]
        rows.append(row)
    return rows


MFMA_FP32_PEAK_TFLOPS = 157.3


def short_kernel_name(name: str) -> str:
    """`void km::(anonymous namespace)::foo<1, 2>(float const*, ...)` -> `foo<1, 2>`."""
    name = name.replace("(anonymous namespace)::", "").replace("km::", "")
    if name.startswith("void "):
        name = name[5:]
    return name.split("(")[0]


def trace_summary(run_dir: str, workload: str, bench_line_file: str) -> str:
    """Markdown summary of one rocprofv3 kernel-trace run of bench.py (see the
    module docstring)."""
    from . import datagen

    cfg = datagen.CONFIGS[workload]
    n, k, d = cfg.n, cfg.k, cfg.d
    flops = 2.0 * n * k * d
    with open(os.path.join(run_dir, "bench_kernel_stats.csv"), newline="") as f:
        stats = list(csv.DictReader(f))
    with open(os.path.join(run_dir, "bench_kernel_trace.csv"), newline="") as f:
        trace = list(csv.DictReader(f))
    bench = None
    with open(bench_line_file) as f:
        for line in f:
            line = line.strip()
            if line.startswith("{") and '"metric"' in line:
                bench = json.loads(line)
    if bench is None:
        raise ValueError(f"no bench.py line in {bench_line_file}")
    total_ns = sum(float(r["TotalDurationNs"]) for r in stats)
    rows = sorted(stats, key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"# Kernel trace — one Lloyd step, {workload} (n={n}, k={k}, d={d}, fp32)", "",
           "Command (on one MI355X; `<repo>` is the repository root):", "",
           f"    cd /tmp && rocprofv3 --kernel-trace --stats --output-format csv -d "
           f"<repo>/gpurun_out/trace_{workload} -o bench -- python3 -u <repo>/bench.py "
           f"--config {workload} --steps 5 --warmup 1 --no-cpu-baseline", "",
           "Summary written by `python3 -m nearest_centroid_assignment_amd.profile_run trace "
           f"--dir <repo>/gpurun_out/trace_{workload} --workload {workload} --bench-line <that "
           "command's stdout>`.", "",
           "bench.py in that mode runs Lloyd steps untimed for at least 300 ms (the GPU's clocks "
           "ramp up over the first tens of ms), then 1 warmup + 5 timed Lloyd steps, then 1 + "
           f"{bench['assign_calls']} assignment-only calls (no min_dist), then one more assignment "
           "and 5 update-only calls back to back. Figures from `bench_kernel_stats.csv` (ns, shown "
           "in µs), averaged over every call. A Lloyd step runs row_sqnorms (centroids), fill_keys "
           "(not where the product kernel stores every key), the assignment's product kernel, "
           "rank_hist fused with finalize (`<true, true>`), the rest of the counting sort (k <= 1024 "
           "and n <= 65536: place, one launch; otherwise tile_prefix, cluster_scan and scatter), "
           "segment_mean with the sample norms (`<..., true>`) and add_norms; a plain update runs "
           "rank_hist on labels (`<true, false>`), the same counting kernels and segment_mean "
           "without norms.", "",
           "| kernel | calls | average (µs) | min (µs) | share |", "|---|---|---|---|---|"]
    for r in rows:
        out.append(f"| {short_kernel_name(r['Name'])} | {r['Calls']} | "
                   f"{float(r['AverageNs']) / 1e3:.1f} | {float(r['MinNs']) / 1e3:.1f} | "
                   f"{100.0 * float(r['TotalDurationNs']) / total_ns:.2f} % |")
    out += ["", "Derived:"]
    prod = [r for r in rows if short_kernel_name(r["Name"]).startswith(ASSIGN_KERNELS)]
    if prod:
        p = prod[0]
        pname = short_kernel_name(p["Name"])
        avg_ms = float(p["AverageNs"]) / 1e6
        out.append(f"* {pname}: 2·n·k·d = {flops:.4e} flop / {avg_ms:.3f} ms = "
                   f"{flops / avg_ms / 1e9:.1f} TFLOP/s = "
                   f"{flops / avg_ms / 1e9 / MFMA_FP32_PEAK_TFLOPS:.3f} of the "
                   f"{MFMA_FP32_PEAK_TFLOPS} TFLOP/s fp32 MFMA peak.")
        disp = sorted((int(r["Dispatch_Id"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
                      for r in trace if r["Kernel_Name"] == p["Name"])
        calls = int(bench["assign_calls"])
        timed = [t for _, t in disp[len(disp) - 1 - calls: len(disp) - 1]]
        if len(timed) == calls and calls > 0:
            t_ms = sum(timed) / len(timed) / 1e6
            out.append(f"* {pname} in the {calls} timed kmeans_assign calls alone (the average "
                       f"above also counts the untimed pre-warm steps): {t_ms * 1e3:.1f} µs = "
                       f"{flops / t_ms / 1e9:.1f} TFLOP/s = "
                       f"{flops / t_ms / 1e9 / MFMA_FP32_PEAK_TFLOPS:.3f} of peak; bench.py's "
                       "assign_ms below also counts the call's small kernels.")
    plain = [r for r in rows if short_kernel_name(r["Name"]).startswith("segment_mean_kernel<")
             and short_kernel_name(r["Name"]).endswith("false>")]
    if plain:
        b = 4.0 * n * d + 4.0 * k * d + 4.0 * n
        t = float(plain[0]["AverageNs"]) / 1e9
        out.append(f"* segment_mean (plain update): {t * 1e6:.1f} µs for 4·n·d + 4·k·d + 4n = "
                   f"{b:.4e} B → {b / t / 1e12:.2f} TB/s.")
    ub = 4.0 * n * d + 8.0 * n + 4.0 * k * d
    out.append(f"* bench.py's line from the same run: Lloyd step {bench['lloyd_ms']:.3f} ms, "
               f"kmeans_assign {bench['assign_ms']:.3f} ms ({bench['assign_tflops']:.1f} TFLOP/s), "
               f"kmeans_update {bench['update_ms']:.3f} ms ({bench['update_hbm_gbps']:.0f} GB/s of "
               f"algorithmic bytes 4nd + 8n + 4kd = {ub:.4e} B).")
    return "\n".join(out) + "\n"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", nargs="?", default="run",
                    choices=["run", "summarize", "kernels", "trace"])
    ap.add_argument("--workload", default="feature_heavy")
    ap.add_argument("--op", default="assign", choices=["assign", "update", "kmeanspp"])
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--out")
    ap.add_argument("--dir", action="append", default=[])
    ap.add_argument("--bench-line")
    a = ap.parse_args(argv)
    if a.mode == "run":
        run(a.workload, a.op)
    elif a.mode == "trace":
        text = trace_summary(a.dir[0], a.workload, a.bench_line)
        if a.out:
            with open(a.out, "w") as f:
                f.write(text)
        else:
            print(text, end="")
    elif a.mode == "summarize":
        print(json.dumps(summarize(a.fetch, a.write, a.out, a.workload), indent=1))
    else:
        for r in kernel_table(a.dir):
            extra = f"  {r['bytes']:.4e} B (x{r['scale']:.3f})" if "bytes" in r else ""
            print(f"{r['kernel'][:90]:90s} {r['counter']:22s} n={r['dispatches']:3d} "
                  f"avg={r['average']:.6g}{extra}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
