"""Host-side logic of bench.py (no GPU needed)."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from nearest_centroid_assignment_amd import datagen  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a configuration that was not measured


def test_traffic_record_requires_matching_kernel(tmp_path, monkeypatch):
    from nearest_centroid_assignment_amd.profile_run import kernel_digest

    cfg = datagen.CONFIGS["feature_heavy"]
    rec = {"workload": "feature_heavy", "beyond_l2_bytes_per_launch": 123.0,
           "assign_kernel_sha256": kernel_digest()}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_record(cfg) == 123.0
    # Another workload, or a kernel changed since the counters were taken.
    assert bench.traffic_record(datagen.CONFIGS["mid"]) is None
    rec["assign_kernel_sha256"] = "0" * 64
    f.write_text(json.dumps(rec))
    assert bench.traffic_record(cfg) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.traffic_record(cfg) is None


def test_cpu_baselines_report_their_sample():
    X, C = datagen.make("tiny")
    b = bench.cpu_baseline(X, C, 0.05)
    assert b["kind"] == "oracle" and b["unit"] == "TFLOP/s" and b["value"] > 0
    assert b["cores"] >= 1 and "rows" in b["sample"]
    assert b["cpus_available"] >= 1 and "omp_num_threads" in b and "cpu_model" in b
    k, trials = 17, 4
    first, rand = datagen.make_seeding_draws(len(X), k, trials)
    p = bench.cpu_baseline_kmeanspp(X, k, first, trials, rand, 0.05)
    assert p["kind"] == "oracle" and p["unit"] == "ms" and p["value"] > 0
    assert "of 17 centres" in p["sample"]


def test_bench_workloads_exist():
    for name in ("feature_heavy", "centroid_heavy", "kmeanspp", "mid"):
        cfg = datagen.CONFIGS[name]
        assert cfg.flops == 2.0 * cfg.n * cfg.k * cfg.d or np.isclose(
            cfg.flops, 2.0 * cfg.n * cfg.k * cfg.d)
    assert set(bench.PAGES_LLOYD_MS) <= set(datagen.CONFIGS)


def test_metric_names_the_workload_shape():
    fh = datagen.CONFIGS["feature_heavy"]
    assert bench.METRIC_FMT.format(n=fh.n, k=fh.k, d=fh.d) == bench.METRIC
    mid = datagen.CONFIGS["mid"]
    assert "65536×1024×2048" in bench.METRIC_FMT.format(n=mid.n, k=mid.k, d=mid.d)


def test_assign_kernel_name_follows_the_tile_rule():
    """The kernel named in the roofline record: DMA-staged 256 x 256 tiles
    for the aligned benchmark shapes and for the ragged shapes where they
    were measured faster than 128 x 256 ones on 256 CUs; the register-staged
    kernel where the 256-row edge or last round wastes more (k = 300,
    50000 x 700), for fewer than 256 tiles, and for rows that are not whole
    16-byte chunks (d not a multiple of 4)."""
    dma, reg, small = "assign_dma_kernel", "assign_tile_kernel", "assign_smallk_kernel"
    for shape in [(512, 17, 64), (1 << 20, 16, 64), (1000, 1, 4), (2000, 64, 192),
                  (513, 16, 960), (1 << 20, 100, 128), (1 << 17, 128, 64)]:
        assert bench.assign_kernel_name(*shape) == small, shape
    # k above 128, above 64 with fewer than 2^17 samples, C past 64 KiB of LDS
    # (64 rows of 256 + 4 floats; 128 rows of 128 + 4), or d not a multiple of
    # 4: not the small-k kernel.
    for shape in [(4096, 65, 64), (1 << 20, 129, 32), (262144, 64, 256), (513, 16, 1024),
                  (4096, 16, 98), (1 << 20, 128, 96)]:
        assert bench.assign_kernel_name(*shape) != small, shape
    for name in ("mid", "feature_heavy", "centroid_heavy", "sample_heavy"):
        cfg = datagen.CONFIGS[name]
        assert bench.assign_kernel_name(cfg.n, cfg.k, cfg.d) == dma
    for shape in [(65000, 1000, 2048), (100000, 1500, 1024), (65536, 4000, 4096),
                  (131000, 8100, 1024), (20000, 5000, 512), (65000, 1024, 2048),
                  (65536, 1024, 96), (65536, 4096, 300), (65536, 4096, 992), (131072, 8192, 96)]:
        assert bench.assign_kernel_name(*shape) == dma, shape
    for shape in [(60000, 300, 2048), (50000, 700, 1024), (4000, 1000, 1024),
                  (65536, 1024, 2050), (65536, 1024, 99), (4096, 256, 512)]:
        assert bench.assign_kernel_name(*shape) == reg, shape
