"""Write the oracle's k-means++ seeding at the pages' seeding shape.

Usage: ``python tests/golden/make_kmeanspp_expected.py``

Draws the seeding workload (65536 samples x 8192 features, blobs; k = 1024
centres, 2 + floor(ln k) = 8 trials per centre, the first centre and the
uniforms from the seeded generator of ``nearest_centroid_assignment_amd.
datagen``, which holds none of the method's arithmetic) and runs
``oracle.kmeanspp`` -- the greedy D^2 seeding in float64, difference-form
distances -- for all k centres. Stores in tests/golden/kmeanspp_seeding.npz:

  chosen      (k,) int64   the oracle's centre indices, in order
  x_sha256    SHA-256 of the bytes of X (the test regenerates X and checks it)
  rand_sha256 SHA-256 of the uniforms
  first, trials, n, k, d, seed

Nothing here calls the GPU library ("004 - tile sizes, a Cython Lloyd step,
and k-means++", section k-means++, for the method and the shape).
"""
from __future__ import annotations

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
from tests.golden.make_full_size_expected import sha256_of  # noqa: E402

PATH = os.path.join(HERE, "kmeanspp_seeding.npz")


def write(seed: int = 0) -> str:
    cfg = datagen.CONFIGS["kmeanspp"]
    X, _ = datagen.make(cfg, seed=seed)
    trials = oracle.default_trials(cfg.k)
    first, rand = datagen.make_seeding_draws(cfg.n, cfg.k, trials, seed=seed)
    t0 = time.time()
    chosen = oracle.kmeanspp(X, cfg.k, first, trials, rand)
    print(f"oracle seeding of {cfg.k} centres: {time.time() - t0:.0f} s on "
          f"{oracle.num_threads()} threads", flush=True)
    np.savez_compressed(PATH, chosen=np.asarray(chosen, dtype=np.int64),
                        x_sha256=np.array(sha256_of(X)), rand_sha256=np.array(sha256_of(rand)),
                        first=np.int64(first), trials=np.int64(trials), n=np.int64(cfg.n),
                        k=np.int64(cfg.k), d=np.int64(cfg.d), seed=np.int64(seed))
    return PATH


if __name__ == "__main__":
    print(write())
