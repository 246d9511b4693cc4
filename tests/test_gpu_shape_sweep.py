"""A seeded sweep of Lloyd steps over random shapes, every assignment tile the
launcher can select (by its own rule, or forced through KMEANS_ASSIGN_TILE,
which falls back where a tile does not apply), against the oracle on every
row under the parity rules of gpu_util. Seven regimes: small k (C resident in
LDS), ragged shapes big enough for the DMA-staged 256 x 256 tiles, whole
multiples of the tiles, tiny odd shapes, many small clusters, anything, and
integer-valued data (exact arithmetic, frequent exact ties, which the lowest
index must win). A quarter of the cases move one centroid far away, so its
cluster is empty and keeps its centre."""
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
