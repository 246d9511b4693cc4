"""Seeded sweeps over random shapes against the oracle. First, Lloyd steps
with every assignment tile the launcher can select (by its own rule, or
forced through KMEANS_ASSIGN_TILE, which falls back where a tile does not
apply), against the oracle on every row under the parity rules of gpu_util. Seven regimes: small k (C resident in
LDS), ragged shapes big enough for the DMA-staged 256 x 256 tiles, whole
multiples of the tiles, tiny odd shapes, many small clusters, anything, and
integer-valued data (exact arithmetic, frequent exact ties, which the lowest
index must win). A quarter of the cases move one centroid far away, so its
cluster is empty and keeps its centre. Then the Lloyd driver (kmeans_fit)
on well-separated data, with and without relocation, k-means++ seeding
with the oracle's draws, and the update on skewed label distributions."""
import numpy as np
import pytest

from tests import gpu_util as gu
from nearest_centroid_assignment_amd import datagen

pytestmark = pytest.mark.gpu

TILES = [None, None, None, "smallk", "256x256", "128x256", "256x128", "128x128", "64x64"]


def _case(i: int, seed0: int = 7100):
    rng = np.random.default_rng(seed0 + i)
    regime = i % 7
    if regime == 0:    # small k
        n, k, d = int(rng.integers(1, 30000)), int(rng.integers(1, 129)), int(rng.integers(1, 400))
    elif regime == 1:  # ragged, DMA-sized
        n, k, d = (int(rng.integers(12000, 40000)), int(rng.integers(300, 1500)),
                   int(4 * rng.integers(1, 150)))
    elif regime == 2:  # whole multiples of the tiles
        n, k, d = (256 * int(rng.integers(1, 120)), 256 * int(rng.integers(1, 6)),
                   64 * int(rng.integers(1, 8)))
    elif regime == 3:  # tiny, odd
        n, k, d = int(rng.integers(1, 600)), int(rng.integers(1, 300)), int(rng.integers(1, 70))
    elif regime == 4:  # many clusters of few rows
        n, k, d = (int(rng.integers(2000, 20000)), int(rng.integers(500, 5000)),
                   int(rng.integers(1, 200)))
    elif regime == 5:  # anything
        n, k, d = int(rng.integers(1, 50000)), int(rng.integers(1, 3000)), int(rng.integers(1, 600))
    else:              # integer-valued
        n, k, d = int(rng.integers(1, 20000)), int(rng.integers(1, 600)), int(rng.integers(1, 257))
    k = max(1, min(k, n))
    if n * k * d > 4e10:
        d = max(1, int(4e10 // (n * k)))
    tile = TILES[int(rng.integers(0, len(TILES)))]
    kb = None if rng.random() < 0.2 else k
    far = bool(rng.random() < 0.25 and k > 1)
    far_at = int(rng.integers(0, k))
    md = bool(rng.random() < 0.8)
    return regime, n, k, d, tile, kb, far, far_at, md


CASES = [_case(i) for i in range(70)]


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}-{c[1]}x{c[2]}x{c[3]}-{c[4]}" for c in CASES])
def test_shape_sweep(monkeypatch, case):
    regime, n, k, d, tile, kb, far, far_at, md = case
    if tile is None:
        monkeypatch.delenv("KMEANS_ASSIGN_TILE", raising=False)
    else:
        monkeypatch.setenv("KMEANS_ASSIGN_TILE", tile)
    gu.announce(f"sweep regime {regime} {n}x{k}x{d} tile={tile} far={far} min_dist={md}")
    seed = n + 7 * k + 13 * d
    if regime == 6:
        X, C = datagen.make_integer(n, k, d, seed=seed)
    else:
        X, C = datagen.make_blobs(n, k, d, kb, 1.0, 0.5, seed=seed)
    if far:
        C = datagen.with_far_centroid(X, C, far_at)
    r = gu.full_parity(X, C, min_dist=md)
    if regime == 6:
        # Exact arithmetic on both sides: the labels, ties included, are equal.
        assert r["mismatches"] == 0


def _fit_case(i: int, seed0: int = 9300):
    """Well-separated blobs (centres 8 sigma apart per feature) with every
    centroid starting near its own blob's centre: no near ties, so the GPU
    driver and the oracle's take the same labels at every iteration. With
    relocation, one to three centroids start far away (empty clusters) and
    one or two iterations run (a relocated centre then splits a blob, whose
    later iterations do have near ties)."""
    rng = np.random.default_rng(seed0 + i)
    n, k, d = int(rng.integers(50, 20000)), int(rng.integers(2, 600)), int(rng.integers(2, 300))
    k = min(k, n)
    relocate = bool(rng.random() < 0.6)
    far = [int(rng.integers(0, k)) for _ in range(int(rng.integers(1, 4)))] \
        if rng.random() < 0.3 else []
    max_iter = int(rng.choice([1, 2])) if relocate else int(rng.choice([1, 2, 5, 20]))
    tol = float(rng.choice([0.0, 1e-4]))
    return n, k, d, relocate, tuple(far), max_iter, tol


FIT_CASES = [_fit_case(i) for i in range(30)]


@pytest.mark.parametrize("case", FIT_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-reloc{int(c[3])}-far{len(c[4])}-it{c[5]}"
                              for c in FIT_CASES])
def test_fit_sweep(case):
    import oracle
    from tests.test_gpu_fit import compare, gpu_fit

    n, k, d, relocate, far, max_iter, tol = case
    gu.announce(f"fit sweep {n}x{k}x{d} relocate={relocate} far={len(far)} max_iter={max_iter}")
    rng = np.random.default_rng(n + 7 * k + 13 * d)
    centres = (8.0 * rng.standard_normal((k, d))).astype(np.float32)
    X = (centres[rng.permutation(np.arange(n) % k)] + rng.standard_normal((n, d))).astype(np.float32)
    C = (centres + 0.3 * rng.standard_normal((k, d))).astype(np.float32)
    for j in far:
        C = datagen.with_far_centroid(X, C, j)
    g = gpu_fit(X, C, max_iter, tol, relocate)
    o = oracle.fit(X, C, max_iter, tol, relocate)
    compare(g, o, X)


def _pp_case(i: int, seed0: int = 9800):
    rng = np.random.default_rng(seed0 + i)
    n, d, k = int(rng.integers(1, 12000)), int(rng.integers(1, 600)), int(rng.integers(1, 200))
    return min(k, n), n, d, int(rng.integers(1, 17)), i % 2 == 0


PP_CASES = [_pp_case(i) for i in range(30)]


@pytest.mark.parametrize("case", PP_CASES,
                         ids=[f"{c[1]}x{c[2]}-k{c[0]}-t{c[3]}-{'int' if c[4] else 'blobs'}"
                              for c in PP_CASES])
def test_kmeanspp_sweep(case):
    """k-means++ seeding with the same draws as the oracle: integer samples
    (every distance and potential exact) and blobs (float64 sums in two
    orders, equal unless a draw falls within rounding of a boundary): the
    chosen indices are equal."""
    import oracle
    from tests.test_gpu_kmeanspp import gpu_pp

    k, n, d, trials, integer = case
    gu.announce(f"kmeans++ sweep {n}x{d} k={k} trials={trials} integer={integer}")
    seed = n + 7 * k + 13 * d
    if integer:
        X, _ = datagen.make_integer(n, 1, min(d, 256), seed=seed)
    else:
        X, _ = datagen.make_blobs(n, 1, d, max(1, min(n, 1 + seed % 49)), 2.0, 1.0, seed=seed)
    first, rand = datagen.make_seeding_draws(n, k, trials, seed=seed)
    C, ch = gpu_pp(X, k, first, trials, rand)
    want = oracle.kmeanspp(X, k, first, trials, rand)
    assert np.array_equal(ch, want)
    assert np.array_equal(C, X[want])


def _update_case(i: int, seed0: int = 10400):
    rng = np.random.default_rng(seed0 + i)
    n, k, d = int(rng.integers(0, 70000)), int(rng.integers(1, 20000)), int(rng.integers(1, 700))
    if n * d > 3e7:
        d = max(1, int(3e7 // max(n, 1)))
    return n, k, d, i % 5


UPDATE_CASES = [_update_case(i) for i in range(30)]
LABEL_KINDS = ("uniform", "zipf", "giant", "few-used", "sorted")


@pytest.mark.parametrize("case", UPDATE_CASES,
                         ids=[f"{c[0]}x{c[1]}x{c[2]}-{LABEL_KINDS[c[3]]}" for c in UPDATE_CASES])
def test_update_sweep(case):
    """kmeans_update on labels it did not compute: uniform, Zipf-skewed (a few
    clusters far above the split size, summed in parts), one cluster holding
    nine rows in ten, a fiftieth of the clusters used (the rest empty, keeping
    their centres) and sorted (each cluster's rows contiguous in X). Counts
    bit-exact, centres per the update rule, bit-exact up to the split size."""
    import torch

    from nearest_centroid_assignment_amd import binding

    n, k, d, kind = case
    gu.announce(f"update sweep {n}x{k}x{d} labels={LABEL_KINDS[kind]}")
    rng = np.random.default_rng(n + 7 * k + 13 * d)
    if n == 0:
        lab = np.zeros(0, np.int64)
    elif kind == 0:
        lab = rng.integers(0, k, n)
    elif kind == 1:
        lab = (rng.zipf(1.3, n) - 1) % k
    elif kind == 2:
        lab = np.where(rng.random(n) < 0.9, int(rng.integers(0, k)), rng.integers(0, k, n))
    elif kind == 3:
        used = rng.choice(k, size=max(1, k // 50), replace=False)
        lab = used[rng.integers(0, len(used), n)]
    else:
        lab = np.sort(rng.integers(0, k, n))
    lab = lab.astype(np.int64)
    X = rng.standard_normal((n, d), dtype=np.float32) + np.float32(rng.uniform(-5, 5))
    C_old = rng.standard_normal((k, d), dtype=np.float32)
    Cg = gu.to_gpu(C_old)
    C_new = torch.empty_like(Cg)
    counts = torch.empty(k, dtype=torch.int64, device=Cg.device)
    binding.kmeans_update(gu.to_gpu(X), gu.to_gpu(lab), Cg, C_new, counts)
    torch.cuda.synchronize()
    gu.check_update(X, lab, C_old, C_new.cpu().numpy(), counts.cpu().numpy())
