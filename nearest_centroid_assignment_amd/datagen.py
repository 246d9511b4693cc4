"""Seeded synthetic inputs for the nearest-centroid assignment / Lloyd update.

This module only draws input arrays. It holds none of the method's arithmetic
(no distance, argmin, sum or mean), so both the GPU path and the float64 CPU
oracle may take their inputs from it without sharing any computation.

The pages ("Three shapes that fit an eager Gram assignment", section Shapes;
"Fusion probe", section Probe shape; "004 - tile sizes, a Cython Lloyd step,
and k-means++", sections Gram tiles on feature-heavy and Same arrays as the
Cython iteration) fix the float32 shapes but never state how X and C were drawn.
The recipe used here is Gaussian blobs:

  1. blob centres (kb, d) = sigma_c * N(0, 1), float32;
  2. membership = a seeded permutation of arange(n) % kb (balanced blobs);
  3. X = centres[membership] + sigma * N(0, 1), float32;
  4. C = X[rows], rows drawn without replacement (k distinct rows of X).

The sample-heavy shape draws X i.i.d. N(0, 1) instead of blobs.

Streams: the membership permutation and the rows of C come from
``numpy.random.default_rng(seed)`` in that order. The normal draws of the
centres and of the noise are split into blocks of 4096 rows; block b of stream
s is drawn from ``numpy.random.default_rng([seed, s, b])`` (s = 1 for the
centres, 2 for the noise), so blocks can be filled by parallel threads and a
seed still names the bytes, whatever the thread count.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Config",
    "CONFIGS",
    "make",
    "make_blobs",
    "make_integer",
    "make_seeding_draws",
    "with_far_centroid",
]


@dataclass(frozen=True)
class Config:
    """A workload: n samples, k centroids, d features (all float32)."""

    name: str
    n: int
    k: int
    d: int
    kb: int | None  # number of Gaussian blobs; None = i.i.d. N(0, sigma^2)
    sigma_c: float  # standard deviation of the blob centres
    sigma: float  # per-feature noise around a blob centre

    @property
    def flops(self) -> float:
        """Algorithmic work of one assignment: the Gram product, 2*n*k*d."""
        return 2.0 * self.n * self.k * self.d


# The workloads. Shapes: Tiny = the n=512, k=17, d=64 label check of the
# fusion probe; Probe = the fusion probe shape; Mid = the shape shared with the
# Cython Lloyd iteration; sample-heavy, centroid-heavy and feature-heavy = the
# three large shapes of the resized-shapes page (the Gram tile grid and the
# Lloyd step of the tile-tradeoff page use feature-heavy). The centroid-heavy
# shape is not printed; it follows from the byte counts printed for it (its
# (n, k) matrix is 4.00 GiB, its Gram tile of 4096 samples 1024 MiB eager, its
# (n, d) difference 2.00 GiB). Its blob parameters are this module's choice
# (one blob per centroid, as for the other blob workloads).
CONFIGS: dict[str, Config] = {
    c.name: c
    for c in (
        Config("tiny", 512, 17, 64, kb=17, sigma_c=4.0, sigma=1.0),
        Config("probe", 4096, 256, 512, kb=256, sigma_c=1.0, sigma=0.5),
        Config("mid", 65536, 1024, 2048, kb=1024, sigma_c=1.0, sigma=0.5),
        Config("sample_heavy", 131072, 8192, 8192, kb=None, sigma_c=0.0, sigma=1.0),
        Config("feature_heavy", 65536, 4096, 16384, kb=4096, sigma_c=1.0, sigma=1.0),
        Config("centroid_heavy", 65536, 16384, 8192, kb=16384, sigma_c=1.0, sigma=1.0),
        # The k-means++ timing shape of the tile-tradeoff page (k = centres to seed).
        Config("kmeanspp", 65536, 1024, 8192, kb=1024, sigma_c=1.0, sigma=1.0),
    )
}


BLOCK_ROWS = 4096


def _fill_normal(seed: int, stream: int, out: np.ndarray, block_rows: int = BLOCK_ROWS) -> None:
    """Fill a (rows, d) float32 array with N(0, 1) draws, block by block.

    Block b (rows [b * block_rows, (b + 1) * block_rows)) is drawn from
    ``default_rng([seed, stream, b])``; blocks are filled by a thread pool.
    """
    rows = out.shape[0]
    starts = list(range(0, rows, block_rows))

    def work(b: int) -> None:
        r0 = starts[b]
        r1 = min(rows, r0 + block_rows)
        np.random.default_rng([seed, stream, b]).standard_normal(
            out[r0:r1].shape, dtype=np.float32, out=out[r0:r1])

    workers = max(1, min(16, os.cpu_count() or 1, len(starts)))
    if workers == 1:
        for b in range(len(starts)):
            work(b)
    else:
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(work, range(len(starts))))


def make_blobs(n: int, k: int, d: int, kb: int | None, sigma_c: float, sigma: float,
               seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Draw (X, C) following the blob recipe in this module's docstring.

    Returns X (n, d) and C (k, d), both C-contiguous float32. Requires k <= n.
    """
    if not (1 <= k <= n) or d < 1:
        raise ValueError(f"need 1 <= k <= n and d >= 1, got n={n} k={k} d={d}")
    rng = np.random.default_rng(seed)
    X = np.empty((n, d), dtype=np.float32)
    if kb is None:
        _fill_normal(seed, 2, X)
        if sigma != 1.0:
            X *= np.float32(sigma)
    else:
        centres = np.empty((kb, d), dtype=np.float32)
        _fill_normal(seed, 1, centres)
        centres *= np.float32(sigma_c)
        membership = rng.permutation(np.arange(n) % kb)
        _fill_normal(seed, 2, X)
        X *= np.float32(sigma)
        for r0 in range(0, n, BLOCK_ROWS):
            r1 = min(n, r0 + BLOCK_ROWS)
            X[r0:r1] += centres[membership[r0:r1]]
    rows = rng.choice(n, size=k, replace=False)
    C = np.ascontiguousarray(X[rows])
    return X, C


def make(config: str | Config, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Draw (X, C) for a named workload (a key of ``CONFIGS``)."""
    cfg = CONFIGS[config] if isinstance(config, str) else config
    return make_blobs(cfg.n, cfg.k, cfg.d, cfg.kb, cfg.sigma_c, cfg.sigma, seed)


def make_seeding_draws(n: int, k: int, trials: int, seed: int = 0) -> tuple[int, np.ndarray]:
    """Random draws consumed by k-means++ seeding: the first centre's index
    (uniform in [0, n)) and (k - 1, trials) float64 uniforms in [0, 1), from
    ``default_rng([seed, 3])`` in that order."""
    rng = np.random.default_rng([seed, 3])
    first = int(rng.integers(0, n))
    return first, rng.random((max(k - 1, 0), trials))


def make_integer(n: int, k: int, d: int, lo: int = -8, hi: int = 8,
                 seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Integer-valued float32 X (n, d) and C (k, d), entries uniform in [lo, hi].

    With |entries| <= 8 and d <= 256 every product and partial sum of the
    distance is an integer below 2**24, so float32 arithmetic on them is exact
    and exact ties between centroids are frequent.
    """
    rng = np.random.default_rng(seed)
    X = rng.integers(lo, hi + 1, size=(n, d)).astype(np.float32)
    C = rng.integers(lo, hi + 1, size=(k, d)).astype(np.float32)
    return X, C


def with_far_centroid(X: np.ndarray, C: np.ndarray, position: int, offset: float = 1.0e3
                      ) -> np.ndarray:
    """Return a copy of C where row ``position`` is moved far from every sample.

    That centroid then wins no sample, which forces an empty cluster.
    """
    C2 = np.array(C, dtype=np.float32, copy=True)
    C2[position] = np.float32(offset) + np.abs(X).max(axis=0)
    return C2
