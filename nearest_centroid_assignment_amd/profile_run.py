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


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("mode", nargs="?", default="run", choices=["run", "summarize", "kernels"])
    ap.add_argument("--workload", default="feature_heavy")
    ap.add_argument("--op", default="assign", choices=["assign", "update", "kmeanspp"])
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--out")
    ap.add_argument("--dir", action="append", default=[])
    a = ap.parse_args(argv)
    if a.mode == "run":
        run(a.workload, a.op)
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
