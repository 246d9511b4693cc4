"""Write the oracle's assignment of EVERY row of the large workloads.

Usage: ``python tests/golden/make_full_size_expected.py [name ...]``
(default: sample_heavy feature_heavy centroid_heavy).

For each workload this draws (X, C) with the seeded generator
(``nearest_centroid_assignment_amd.datagen``, which holds none of the method's
arithmetic) and runs ``oracle.assign`` -- the float64 difference-form distance
with the lowest index winning exact ties -- on all n rows against all k
centroids. It stores, in ``tests/golden/full_<name>.npz``:

  labels  (n,) int32    the oracle's label of every row
  best    (n,) float64  its distance D_i,label
  second  (n,) float64  the second-smallest distance over the other centroids
  x_sha256, c_sha256    SHA-256 of the bytes of X and C, so a test can prove
                        it regenerated the same inputs before comparing
  n, k, d, seed

Nothing here calls the GPU library: every stored value comes from ``oracle/``.
The GPU tests (tests/test_gpu_full_size.py) compare the HIP path with these
values on every row, under the parity rules of the near-tie band ("004 - tile
sizes, a Cython Lloyd step, and k-means++", section Same arrays as the Cython
iteration: two float32 implementations may disagree on a row that is a near
tie).
"""
from __future__ import annotations

import hashlib
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from nearest_centroid_assignment_amd import datagen  # noqa: E402

DEFAULT = ("sample_heavy", "feature_heavy", "centroid_heavy")
ROWS_PER_CALL = 4096  # oracle rows per call, so progress can be printed


def path_for(name: str) -> str:
    return os.path.join(HERE, f"full_{name}.npz")


def sha256_of(a: np.ndarray) -> str:
    h = hashlib.sha256()
    flat = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    step = 1 << 28
    for o in range(0, flat.size, step):
        h.update(flat[o:o + step])
    return h.hexdigest()


def write(name: str, seed: int = 0) -> str:
    cfg = datagen.CONFIGS[name]
    t0 = time.time()
    X, C = datagen.make(name, seed=seed)
    print(f"{name}: inputs {X.shape} x {C.shape} drawn in {time.time() - t0:.1f} s", flush=True)
    n = X.shape[0]
    labels = np.empty(n, dtype=np.int32)
    best = np.empty(n, dtype=np.float64)
    second = np.empty(n, dtype=np.float64)
    t0 = time.time()
    for r0 in range(0, n, ROWS_PER_CALL):
        r1 = min(n, r0 + ROWS_PER_CALL)
        lab, b, s = oracle.assign(X[r0:r1], C)
        labels[r0:r1], best[r0:r1], second[r0:r1] = lab, b, s
        el = time.time() - t0
        print(f"{name}: rows {r1}/{n}, {el:.0f} s, about {el / r1 * (n - r1):.0f} s left",
              flush=True)
    out = path_for(name)
    np.savez_compressed(out, labels=labels, best=best, second=second,
                        x_sha256=np.array(sha256_of(X)), c_sha256=np.array(sha256_of(C)),
                        n=np.int64(cfg.n), k=np.int64(cfg.k), d=np.int64(cfg.d),
                        seed=np.int64(seed))
    print(f"{name}: wrote {out} ({os.path.getsize(out) / 2**20:.2f} MiB), oracle "
          f"{time.time() - t0:.0f} s on {oracle.num_threads()} threads", flush=True)
    return out


if __name__ == "__main__":
    for nm in (sys.argv[1:] or DEFAULT):
        write(nm)
