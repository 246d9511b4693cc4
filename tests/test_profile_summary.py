"""The kernel-trace summarizer behind profiles/lloyd_*_kernel_trace.md, on a
small fabricated rocprofv3 output (host only)."""
import csv
import json

from nearest_centroid_assignment_amd import datagen
from nearest_centroid_assignment_amd.profile_run import short_kernel_name, trace_summary

PROD = ("void km::(anonymous namespace)::assign_dma_kernel<0>(float const*, float const*, "
        "float const*, long, long, long, int, int, unsigned long long*, int const*)")
MEAN = "void km::(anonymous namespace)::segment_mean_kernel<true, false, 8, false>(float const*)"
NORM = "void km::(anonymous namespace)::segment_mean_kernel<true, false, 8, true>(float const*)"
FILL = "km::(anonymous namespace)::fill_keys_kernel(unsigned long long*, long, km::Gate)"


def test_short_kernel_name():
    assert short_kernel_name(PROD) == "assign_dma_kernel<0>"
    assert short_kernel_name(FILL) == "fill_keys_kernel"
    assert short_kernel_name(
        "void km::(anonymous namespace)::assign_tile_kernel<km::(anonymous namespace)::"
        "TileCfg<2, 2, 1, 1, 32>, 2, 4, false>(float const*)") == \
        "assign_tile_kernel<TileCfg<2, 2, 1, 1, 32>, 2, 4, false>"


def _write(tmp_path, durations_ns, assign_calls):
    # Product-kernel dispatches in launch order: untimed ones, then the timed
    # assignment calls, then the one assignment before the updates.
    trace = [{"Dispatch_Id": i + 1, "Kernel_Name": PROD, "Start_Timestamp": 1000 * i,
              "End_Timestamp": 1000 * i + t} for i, t in enumerate(durations_ns)]
    trace.append({"Dispatch_Id": 999, "Kernel_Name": MEAN, "Start_Timestamp": 0,
                  "End_Timestamp": 800_000})
    with open(tmp_path / "bench_kernel_trace.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(trace[0].keys()))
        w.writeheader()
        w.writerows(trace)
    total = sum(durations_ns)
    stats = [
        {"Name": PROD, "Calls": len(durations_ns), "TotalDurationNs": total,
         "AverageNs": total / len(durations_ns), "MinNs": min(durations_ns)},
        {"Name": MEAN, "Calls": 1, "TotalDurationNs": 800_000, "AverageNs": 800_000,
         "MinNs": 800_000},
        {"Name": NORM, "Calls": 2, "TotalDurationNs": 1_700_000, "AverageNs": 850_000,
         "MinNs": 840_000},
    ]
    with open(tmp_path / "bench_kernel_stats.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(stats[0].keys()))
        w.writeheader()
        w.writerows(stats)
    line = {"metric": "m", "assign_calls": assign_calls, "lloyd_ms": 58.5, "assign_ms": 57.5,
            "assign_tflops": 153.0, "update_ms": 0.87, "update_hbm_gbps": 5250.0}
    (tmp_path / "bench.out").write_text("[bench] log line\n" + json.dumps(line) + "\n")


def test_trace_summary_table_and_rates(tmp_path):
    cfg = datagen.CONFIGS["feature_heavy"]
    flops = 2.0 * cfg.n * cfg.k * cfg.d
    # 3 untimed calls at 60 ms, 2 timed at 57 ms, 1 final at 70 ms.
    durs = [60_000_000] * 3 + [57_000_000] * 2 + [70_000_000]
    _write(tmp_path, durs, assign_calls=2)
    text = trace_summary(str(tmp_path), "feature_heavy", str(tmp_path / "bench.out"))
    lines = text.splitlines()
    rows = [ln for ln in lines if ln.startswith("| ") and not ln.startswith("| kernel")]
    # Sorted by total time: the product kernel, then the norms instance, then the plain one.
    assert [r.split(" | ")[0][2:] for r in rows] == [
        "assign_dma_kernel<0>", "segment_mean_kernel<true, false, 8, true>",
        "segment_mean_kernel<true, false, 8, false>"]
    avg_ms = sum(durs) / len(durs) / 1e6
    assert f"{flops / avg_ms / 1e9 / 157.3:.3f} of the 157.3" in text
    # The timed calls are the two before the last dispatch: 57 ms each.
    assert f"in the 2 timed kmeans_assign calls alone" in text
    assert f"57000.0 µs = {flops / 57.0 / 1e9:.1f} TFLOP/s" in text
    # The plain update's mean kernel (last template argument false): 0.8 ms.
    b = 4.0 * cfg.n * cfg.d + 4.0 * cfg.k * cfg.d + 4.0 * cfg.n
    assert f"800.0 µs for 4·n·d + 4·k·d + 4n = {b:.4e} B → {b / 0.8e-3 / 1e12:.2f} TB/s" in text
    assert "Lloyd step 58.500 ms" in text and "kmeans_update 0.870 ms" in text
