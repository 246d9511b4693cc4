"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Sizes span several 128 x 128 tiles with ragged tails in n, k and d; the
integer-valued cases make float32 arithmetic exact, so there labels (ties
included), counts, centroids and distances must be bit-exact.
"""
import numpy as np
import pytest

import oracle
from nearest_centroid_assignment_amd import datagen
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from nearest_centroid_assignment_amd import binding

    binding.lib()  # fails loudly if the HIP library is missing


@pytest.mark.parametrize("name", ["tiny", "probe"])
def test_small_config_lloyd(name):
    gu.announce(f"lloyd parity {name}")
    X, C = datagen.make(name)
    res = gu.full_parity(X, C)
    assert res["mismatches"] <= res["near_ties"]
    gu.announce(f"{name} near-ties {res['near_ties']} mismatches {res['mismatches']}")


def test_mid_lloyd():
    gu.announce("lloyd parity mid 65536x1024x2048")
    X, C = datagen.make("mid")
    res = gu.full_parity(X, C)
    gu.announce(f"mid near-ties {res['near_ties']} mismatches {res['mismatches']}")


ODD_SHAPES = [
    (1, 1, 1),
    (7, 3, 5),
    (5, 9, 3),          # k > n: some clusters must be empty
    (130, 129, 33),     # one past a tile in n and k, d not a multiple of 4
    (300, 1, 17),       # k = 1
    (257, 200, 1),      # d = 1
    (384, 384, 8),      # k = n
    (333, 65, 1030),    # d past one 1024-column update chunk, d % 4 != 0
    (1000, 300, 1028),  # vector path with a ragged 32-feature stage
    (2049, 130, 96),
]


@pytest.mark.parametrize("n,k,d", ODD_SHAPES, ids=[f"{n}x{k}x{d}" for n, k, d in ODD_SHAPES])
def test_odd_shapes(n, k, d):
    gu.announce(f"odd shape {n}x{k}x{d}")
    rng = np.random.default_rng(n * 7 + k * 13 + d)
    X = rng.standard_normal((n, d), dtype=np.float32)
    C = rng.standard_normal((k, d), dtype=np.float32)
    gu.full_parity(X, C)


def _random_shapes(count=24, seed=2024):
    """Two in three log-uniform in n < 3000, k < 700, d < 700 (degenerate and
    tiny edges), one in three uniform in [200, 3000) x [100, 700) x [100, 700)
    (several tiles and stages with ragged ends)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        if i % 3 == 2:
            out.append(tuple(int(rng.integers(lo, hi)) for lo, hi in ((200, 3000), (100, 700),
                                                                       (100, 700))))
        else:
            out.append(tuple(int(np.exp(rng.uniform(0.0, np.log(hi)))) for hi in (3000, 700, 700)))
    return out


RANDOM_SHAPES = _random_shapes()


@pytest.mark.parametrize("n,k,d", RANDOM_SHAPES, ids=[f"{n}x{k}x{d}" for n, k, d in RANDOM_SHAPES])
def test_random_shapes(n, k, d):
    """Seeded blobs with a common offset (so the Gram form cancels), centres
    drawn from the samples when k <= n (rows at distance 0) or at random."""
    gu.announce(f"random shape {n}x{k}x{d}")
    rng = np.random.default_rng(n + 31 * k + 977 * d)
    kb = max(1, min(k, 40))
    centres = 3.0 * rng.standard_normal((kb, d))
    offset = rng.uniform(-10.0, 10.0, d)
    X = (centres[rng.integers(0, kb, n)] + rng.standard_normal((n, d)) + offset).astype(np.float32)
    if k <= n and rng.random() < 0.5:
        C = X[rng.choice(n, k, replace=False)].copy()
    else:
        C = (3.0 * rng.standard_normal((k, d)) + offset).astype(np.float32)
    gu.full_parity(X, C)


# The Lloyd step gathers the sample norms inside the update when
# ceil(d / 256) * 16 <= k, else it takes a separate pass over X.
NORM_PATHS = [
    (3000, 20, 130, "gathered, scalar loads, clusters of ~150 rows"),
    (3000, 32, 256, "gathered, 16-byte loads, clusters of ~94 rows"),
    (2000, 64, 1024, "gathered, 4 chunks"),
    (2000, 63, 1024, "separate pass (4 chunks * 16 > 63)"),
    (700, 5, 300, "separate pass, k < 16"),
]


@pytest.mark.parametrize("n,k,d,what", NORM_PATHS, ids=[f"{n}x{k}x{d}" for n, k, d, _ in NORM_PATHS])
def test_lloyd_min_dist_paths(n, k, d, what):
    """min_dist of the Lloyd step on both of its paths: against the oracle
    within the tolerance, and against kmeans_assign's min_dist (a separate
    norm pass) to float32 rounding of ||x||^2."""
    gu.announce(f"lloyd min_dist {n}x{k}x{d} ({what})")
    rng = np.random.default_rng(n + k + d)
    centres = 2.0 * rng.standard_normal((k, d))
    X = (centres[rng.integers(0, k, n)] + rng.standard_normal((n, d))).astype(np.float32)
    C = X[rng.choice(n, k, replace=False)].copy()
    res = gu.full_parity(X, C)
    assert res["mismatches"] <= res["near_ties"]
    l_labels, l_md, _, _ = gu.gpu_lloyd(X, C)
    a_labels, a_md = gu.gpu_assign(X, C)
    assert np.array_equal(l_labels, a_labels)
    xn = np.einsum("ij,ij->i", X.astype(np.float64), X.astype(np.float64))
    # Both add a float32 ||x||^2 (each within ~1e-6 relative) to the same best
    # value, so they differ by at most a few float32 ulps of ||x||^2.
    assert np.all(np.abs(l_md.astype(np.float64) - a_md) <= 4e-6 * xn + 1e-6)


# Shapes where the launcher's own rule (no forced tile) takes the DMA-staged
# kernel's ragged instances: n not a multiple of 256 with d a multiple of 64,
# and d a multiple of 4 only (a partial last stage).
DMA_DEFAULT = [(65000, 1024, 128), (20000, 3000, 100), (40000, 2000, 300)]
# The small-k kernel in a whole Lloyd step (labels, min_dist, update).
SMALLK_LLOYD = [(20000, 10, 64), (65536, 50, 96), (3001, 64, 192)]


@pytest.mark.parametrize("n,k,d", SMALLK_LLOYD, ids=[f"{n}x{k}x{d}" for n, k, d in SMALLK_LLOYD])
def test_lloyd_smallk(n, k, d):
    """The whole Lloyd step, every row against the oracle, at k <= 64."""
    gu.announce(f"lloyd smallk {n}x{k}x{d}")
    rng = np.random.default_rng(n + k + d)
    centres = 2.0 * rng.standard_normal((k, d))
    X = (centres[rng.integers(0, k, n)] + rng.standard_normal((n, d))).astype(np.float32)
    C = X[rng.choice(n, k, replace=False)].copy()
    res = gu.full_parity(X, C)
    assert res["mismatches"] <= res["near_ties"]


@pytest.mark.parametrize("n,k,d", DMA_DEFAULT, ids=[f"{n}x{k}x{d}" for n, k, d in DMA_DEFAULT])
def test_lloyd_dma_ragged_default(n, k, d):
    """The whole Lloyd step, every row against the oracle, on shapes that the
    default selection sends to the ragged DMA instances (the host-side mirror
    of the rule confirms the choice for a 256-CU device)."""
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    assert bench.assign_kernel_name(n, k, d) == "assign_dma_kernel"
    gu.announce(f"lloyd dma ragged default {n}x{k}x{d}")
    rng = np.random.default_rng(n + k + d)
    centres = 2.0 * rng.standard_normal((k, d))
    X = (centres[rng.integers(0, k, n)] + rng.standard_normal((n, d))).astype(np.float32)
    C = X[rng.choice(n, k, replace=False)].copy()
    res = gu.full_parity(X, C)
    assert res["mismatches"] <= res["near_ties"]


# The counting sort's paths by k: the cluster scan holds 1, 2, 4, 8 or 16
# clusters per thread in registers up to k = 16384 and takes 1024-cluster
# chunks above; the per-tile label table sits in LDS up to k = 16384 and in the
# tile's global histogram column above; more than 64 sort tiles of 1024 rows
# take the batched tile prefix.
COUNT_PATHS = [
    (30000, 1025, 8, "2 clusters per thread, 2 scan blocks"),
    (66000, 2049, 8, "4 per thread, 65 sort tiles"),
    (30000, 8193, 8, "16 per thread, 9 scan blocks"),
    (20000, 16385, 8, "global label table, chunked scan"),
    (12000, 40000, 4, "k > n: global table, chunked scan, 40 scan blocks"),
]


@pytest.mark.parametrize("n,k,d,what", COUNT_PATHS,
                         ids=[f"{n}x{k}x{d}" for n, k, d, _ in COUNT_PATHS])
def test_lloyd_count_paths(n, k, d, what):
    """The whole Lloyd step (labels from the assignment's packed keys) on every
    row, at k on each side of the counting sort's limits."""
    gu.announce(f"lloyd count path {n}x{k}x{d} ({what})")
    rng = np.random.default_rng(n ^ k)
    X = rng.standard_normal((n, d), dtype=np.float32)
    C = rng.standard_normal((k, d), dtype=np.float32)
    res = gu.full_parity(X, C)
    assert res["mismatches"] <= res["near_ties"]


@pytest.mark.parametrize("n,k,d", [(50000, 20000, 33), (70000, 17000, 16), (3000, 16384, 8)])
def test_update_count_paths(n, k, d):
    """kmeans_update on given labels (the other entry to the counting sort)
    with k at and above the LDS table limit, up to 69 sort tiles."""
    from nearest_centroid_assignment_amd import binding
    import torch

    gu.announce(f"update count path {n}x{k}x{d}")
    rng = np.random.default_rng(n + 3 * k)
    X = rng.standard_normal((n, d), dtype=np.float32)
    C = rng.standard_normal((k, d), dtype=np.float32)
    labels = rng.integers(0, k, size=n).astype(np.int64)
    C_new, counts = binding.update(gu.to_gpu(X), gu.to_gpu(labels), gu.to_gpu(C))
    torch.cuda.synchronize()
    counts = counts.cpu().numpy()
    assert np.array_equal(counts, np.bincount(labels, minlength=k))
    gu.check_update(X, labels, C, C_new.cpu().numpy(), counts)


@pytest.mark.parametrize("n,k,d", [(500, 37, 64), (1500, 260, 256), (129, 130, 12)])
def test_integer_exact(n, k, d):
    """|values| <= 8, d <= 256: every float32 product and partial sum is an
    exact integer, so the GPU must match the oracle bit for bit, exact ties
    (duplicate centroids) included."""
    gu.announce(f"integer exact {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=n + k)
    C[k - 1] = C[0]  # duplicate: index 0 must win every such tie
    C[k // 2] = C[1]
    g_labels, g_md, g_Cnew, g_counts = gu.gpu_lloyd(X, C)
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(g_labels, o_labels)
    assert np.array_equal(g_md.astype(np.float64), best)
    C_ref, cnt_ref, _ = oracle.update(X, o_labels, C)
    assert np.array_equal(g_counts, cnt_ref)
    assert np.array_equal(g_Cnew.view(np.uint32), C_ref.view(np.uint32))
    assert not np.any(g_labels == k - 1)


def test_forced_empty_cluster():
    """A centroid far from every sample wins nothing and keeps its position."""
    gu.announce("empty cluster mid-sized")
    X, C = datagen.make_blobs(20000, 300, 128, kb=300, sigma_c=1.0, sigma=0.5, seed=3)
    C = datagen.with_far_centroid(X, C, 123)
    res = gu.full_parity(X, C)
    g_labels, _, g_Cnew, g_counts = gu.gpu_lloyd(X, C)
    assert g_counts[123] == 0
    assert np.array_equal(g_Cnew[123], C[123])


def test_mid_forced_empty_cluster():
    gu.announce("empty cluster on the mid workload")
    X, C = datagen.make("mid")
    C = datagen.with_far_centroid(X, C, 777)
    gu.full_parity(X, C)


def test_in_place_update():
    import torch

    from nearest_centroid_assignment_amd import binding

    gu.announce("in-place update")
    X, C = datagen.make("probe")
    C = datagen.with_far_centroid(X, C, 5)
    Xg, Cg = gu.to_gpu(X), gu.to_gpu(C)
    labels = torch.empty(len(X), dtype=torch.int64, device="cuda:0")
    counts = torch.empty(len(C), dtype=torch.int64, device="cuda:0")
    binding.kmeans_lloyd_step(Xg, Cg, labels, None, Cg, counts)
    torch.cuda.synchronize()
    gu.check_update(X, labels.cpu().numpy(), C, Cg.cpu().numpy(), counts.cpu().numpy())


@pytest.mark.parametrize("n,k,d", [(3000, 40, 70), (70000, 40, 70), (5000, 2000, 70),
                                   (5000, 20000, 16)])
def test_update_ignores_invalid_labels(n, k, d):
    """Rows labelled -1 or k + 3 are left out of every count and sum, on each
    counting path (one launch; four with 69 sort tiles; two clusters per
    scan thread; the global label table)."""
    import torch

    from nearest_centroid_assignment_amd import binding

    gu.announce(f"update with out-of-range labels {n}x{k}x{d}")
    rng = np.random.default_rng(9)
    X = rng.standard_normal((n, d), dtype=np.float32)
    C = rng.standard_normal((k, d), dtype=np.float32)
    labels = rng.integers(0, k, size=n)
    bad = rng.random(n) < 0.1
    labels[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, k + 3)
    C_new, counts = binding.update(gu.to_gpu(X), gu.to_gpu(labels), gu.to_gpu(C))
    torch.cuda.synchronize()
    keep = ~bad
    gu.check_update(X[keep], labels[keep], C, C_new.cpu().numpy(), counts.cpu().numpy())


@pytest.mark.parametrize("k", [17, 2000, 17000])
def test_update_with_no_samples(k):
    """n = 0 on each counting path (one launch for k <= 1024, the tile prefix
    and cluster scan above, chunked above 16384): every cluster is empty and
    keeps its centre, in kmeans_update and in a Lloyd step."""
    import torch

    from nearest_centroid_assignment_amd import binding

    gu.announce(f"update with n = 0, k = {k}")
    C = np.random.default_rng(1).standard_normal((k, 9), dtype=np.float32)
    X = torch.empty((0, 9), dtype=torch.float32, device="cuda:0")
    labels = torch.empty((0,), dtype=torch.int64, device="cuda:0")
    C_new, counts = binding.update(X, labels, gu.to_gpu(C))
    torch.cuda.synchronize()
    assert np.all(counts.cpu().numpy() == 0)
    assert np.array_equal(C_new.cpu().numpy(), C)
    md = torch.empty((0,), dtype=torch.float32, device="cuda:0")
    C_new2 = torch.full((k, 9), float("nan"), dtype=torch.float32, device="cuda:0")
    counts2 = torch.full((k,), -1, dtype=torch.int64, device="cuda:0")
    binding.kmeans_lloyd_step(X, gu.to_gpu(C), labels, md, C_new2, counts2)
    torch.cuda.synchronize()
    assert np.all(counts2.cpu().numpy() == 0)
    assert np.array_equal(C_new2.cpu().numpy(), C)


def test_unaligned_inputs_take_scalar_path():
    """Contiguous views that are not 16-byte aligned use the scalar loads."""
    import torch

    from nearest_centroid_assignment_amd import binding

    gu.announce("unaligned inputs")
    X, C = datagen.make("probe")
    n, d = X.shape
    k = C.shape[0]
    Xs = torch.empty(n * d + 1, dtype=torch.float32, device="cuda:0")[1:].view(n, d)
    Cs = torch.empty(k * d + 3, dtype=torch.float32, device="cuda:0")[3:].view(k, d)
    Xs.copy_(gu.to_gpu(X))
    Cs.copy_(gu.to_gpu(C))
    labels, md, C_new, counts = binding.lloyd_step(Xs, Cs)
    torch.cuda.synchronize()
    ref = gu.gpu_lloyd(X, C)
    assert np.array_equal(labels.cpu().numpy(), ref[0])
    assert np.array_equal(C_new.cpu().numpy(), ref[2])
    assert np.array_equal(counts.cpu().numpy(), ref[3])


def test_deterministic_bits():
    gu.announce("determinism on mid")
    X, C = datagen.make("mid")
    a = gu.gpu_lloyd(X, C)
    b = gu.gpu_lloyd(X, C)
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8))


def test_library_allocates_nothing():
    """With outputs and workspace allocated up front, a Lloyd step on the mid
    workload raises the torch allocator's peak by nothing, and the workspace is
    far below both the (n, k) distance matrix and the (n, d) sample matrix."""
    import torch

    from nearest_centroid_assignment_amd import binding

    gu.announce("allocation accounting")
    cfg = datagen.CONFIGS["mid"]
    X, C = datagen.make("mid")
    Xg, Cg = gu.to_gpu(X), gu.to_gpu(C)
    n, k, d = cfg.n, cfg.k, cfg.d
    labels = torch.empty(n, dtype=torch.int64, device="cuda:0")
    md = torch.empty(n, dtype=torch.float32, device="cuda:0")
    C_new = torch.empty_like(Cg)
    counts = torch.empty(k, dtype=torch.int64, device="cuda:0")
    wsb = binding.kmeans_workspace_bytes(n, k, d, binding.KM_OP_LLOYD)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda:0")
    free_before = torch.cuda.mem_get_info()[0]
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    binding.kmeans_lloyd_step(Xg, Cg, labels, md, C_new, counts, workspace=ws)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == base
    assert torch.cuda.mem_get_info()[0] >= free_before - (64 << 20)
    assert wsb < n * k * 4 / 64 and wsb < n * d * 4 / 64


@pytest.mark.parametrize("tile", ["256x256", "128x256", "256x128", "128x128", "64x64"])
@pytest.mark.parametrize("n,k,d", [(1000, 300, 1028), (130, 129, 33), (2048, 512, 256),
                                   (777, 260, 64), (512, 256, 48), (300, 260, 150),
                                   (257, 130, 100), (260, 257, 16)])
def test_tile_variants(monkeypatch, tile, n, k, d):
    """Every tile shape the launcher can select, on full, ragged and scalar
    paths (integer data: bit-exact labels, ties included). The feature counts
    give 1 to 65 stages, so the main loop runs zero, one or many times and
    every length of the pipeline's tail (1 to 4 stages) occurs."""
    monkeypatch.setenv("KMEANS_ASSIGN_TILE", tile)
    gu.announce(f"tile {tile} {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=n + d)
    C[k - 1] = C[2]
    if d > 64:
        X = X / np.float32(4.0)  # still exact: quarter-integers, small sums
        C = C / np.float32(4.0)
    g_labels, g_md = gu.gpu_assign(X, C)
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(g_labels, o_labels)
    assert np.array_equal(g_md.astype(np.float64), best)


@pytest.mark.parametrize("n,k,d", [(9472, 2304, 64), (1792, 1280, 128), (16384, 4096, 64)])
def test_dma_tile_walk(monkeypatch, n, k, d):
    """The DMA-staged 256 x 256 kernel (operands moved from global memory
    straight into LDS): 333 tiles (more than the CUs, not a multiple of 8),
    35 tiles (fewer than the CUs) and 1024 tiles (four per block). Integer
    data: labels and distances bit-exact."""
    monkeypatch.setenv("KMEANS_ASSIGN_TILE", "256x256")
    gu.announce(f"dma walk {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=n + k + d + 1)
    C[k - 1] = C[5]
    g_labels, g_md = gu.gpu_assign(X, C)
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(g_labels, o_labels)
    assert np.array_equal(g_md.astype(np.float64), best)


@pytest.mark.parametrize("n,k,d", [(9000, 2100, 128), (1000, 300, 64), (70, 17, 64),
                                   (16385, 4095, 64), (5000, 1000, 1024), (300, 1, 64),
                                   (2048, 700, 192), (700, 2048, 64),
                                   (9000, 2100, 96), (4096, 1024, 160), (2048, 512, 784),
                                   (1000, 300, 100), (5000, 1000, 300), (777, 260, 28),
                                   (70, 17, 4), (4096, 512, 20)])
def test_dma_tile_ragged(monkeypatch, n, k, d):
    """The DMA-staged 256 x 256 kernel's ragged instance: edge tiles where
    part of a wave's 64 rows, or all of them, lie past n or k (9000 x 2100:
    the last tiles keep 40 samples and 52 centroids), 324 tiles down to one
    (70 x 17: fewer rows than one wave loads), a single centroid, ragged n or
    k alone; and feature counts that are not a multiple of 64: an odd number
    of 32-feature stages (96, 160, 784), a last stage that ends inside the
    rows (100, 300, 784: 1, 3 and 4 of its 8 chunks), a single partial
    stage (28, 20, 4 features), with whole tiles (4096 x 1024, 2048 x 512)
    or ragged ones. Integer data: labels and distances bit-exact."""
    monkeypatch.setenv("KMEANS_ASSIGN_TILE", "256x256")
    gu.announce(f"dma ragged {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=n + 2 * k + d)
    if k > 6:
        C[k - 1] = C[5]
    g_labels, g_md = gu.gpu_assign(X, C)
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(g_labels, o_labels)
    assert np.array_equal(g_md.astype(np.float64), best)


SMALLK = [(1000, 1, 4), (1000, 5, 60), (4097, 16, 64), (3000, 17, 100), (5000, 33, 128),
          (2000, 64, 192), (777, 48, 320), (513, 16, 960), (70, 3, 36), (40000, 20, 32),
          (131072, 65, 60), (140000, 96, 100), (131072, 100, 128), (131075, 128, 64)]


@pytest.mark.parametrize("n,k,d", SMALLK, ids=[f"{n}x{k}x{d}" for n, k, d in SMALLK])
def test_smallk_kernel(n, k, d):
    """The small-k kernel (C resident in LDS, X streamed into 16 x 16 x 4
    MFMAs), which the launcher takes for these shapes: one to eight 16-row
    blocks of C (k above 64 from 2^17 samples) with rows past k, a last 16-sample group past n (1000, 4097,
    777, 513, 70 samples), features past d in the last 64-feature load (4 to
    960 features), many groups per wave (40000). Integer data with duplicate
    centroids: labels (lowest index on ties) and distances bit-exact."""
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    assert bench.assign_kernel_name(n, k, d) == "assign_smallk_kernel"
    gu.announce(f"smallk {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=n + 3 * k + d)
    if k > 2:
        C[k - 1] = C[1]
    g_labels, g_md = gu.gpu_assign(X, C)
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(g_labels, o_labels)
    assert np.array_equal(g_md.astype(np.float64), best)


def test_smallk_unaligned_falls_back():
    """Samples that are not 16-byte aligned: the small-k shape runs on the
    register-staged kernel instead (scalar loads), with the same results."""
    import torch
    from nearest_centroid_assignment_amd import binding

    n, k, d = 3000, 16, 64
    gu.announce(f"smallk fallback unaligned {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=78)
    flat = torch.zeros(n * d + 1, dtype=torch.float32, device="cuda:0")
    Xg = flat[1:].view(n, d)
    Xg.copy_(torch.from_numpy(X))
    assert Xg.data_ptr() % 16 != 0
    labels, md = binding.assign(Xg, gu.to_gpu(C))
    torch.cuda.synchronize()
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(labels.cpu().numpy(), o_labels)
    assert np.array_equal(md.cpu().numpy().astype(np.float64), best)


def test_dma_tile_unaligned_falls_back(monkeypatch):
    """A 256 x 256 shape whose samples are not 16-byte aligned runs on the
    register-staged kernel instead (scalar loads), with the same results."""
    import torch
    from nearest_centroid_assignment_amd import binding

    monkeypatch.setenv("KMEANS_ASSIGN_TILE", "256x256")
    n, k, d = 2048, 512, 128
    gu.announce(f"dma fallback unaligned {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=77)
    flat = torch.zeros(n * d + 1, dtype=torch.float32, device="cuda:0")
    Xg = flat[1:].view(n, d)
    Xg.copy_(torch.from_numpy(X))
    assert Xg.data_ptr() % 16 != 0
    labels, md = binding.assign(Xg, gu.to_gpu(C))
    torch.cuda.synchronize()
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(labels.cpu().numpy(), o_labels)
    assert np.array_equal(md.cpu().numpy().astype(np.float64), best)


@pytest.mark.parametrize("tile", ["128x256", "256x128"])
@pytest.mark.parametrize("n,k,d", [(9472, 1280, 64), (1792, 640, 96), (33024, 1280, 32)])
def test_persistent_tile_walk(monkeypatch, tile, n, k, d):
    """Full tiles of the 512-thread shapes run as one persistent block per
    CU walking its XCD's tiles: 370 tiles (more than the CUs, not a multiple
    of 8), 35 tiles (fewer than the CUs) and 1290 tiles (several per block,
    uneven XCD ranges). Integer data: labels and distances bit-exact."""
    monkeypatch.setenv("KMEANS_ASSIGN_TILE", tile)
    gu.announce(f"persistent walk {tile} {n}x{k}x{d}")
    X, C = datagen.make_integer(n, k, d, seed=n + k + d)
    C[k - 1] = C[3]
    g_labels, g_md = gu.gpu_assign(X, C)
    o_labels, best, _ = oracle.assign(X, C)
    assert np.array_equal(g_labels, o_labels)
    assert np.array_equal(g_md.astype(np.float64), best)


@pytest.mark.parametrize("n,k,d,skew", [(5000, 3, 300, "mild"), (70000, 2, 520, "giant"),
                                        (20000, 50, 1030, "zipf"), (3000, 200, 64, "one-big"),
                                        (70125, 375, 512, "ramp"), (70125, 375, 1024, "ramp"),
                                        (65536, 2048, 1024, "edge")])
def test_update_skewed_clusters(n, k, d, skew):
    """Cluster sizes far from balanced: big clusters take the split-row path,
    small ones the in-order path; both must meet the update rules. The ramp
    (cluster j holds j rows, shuffled) covers every size from empty to 374 on
    both sides of the 2^26-element line where the one-wave path grows from
    64 to 128 rows; "edge" sits exactly on that line and on n = 32 k (both
    inclusive), with clusters of 0 to 255 rows and the rest of about 18."""
    from nearest_centroid_assignment_amd import binding
    import torch

    gu.announce(f"skewed update {skew} {n}x{k}x{d}")
    rng = np.random.default_rng(n + k)
    X = rng.standard_normal((n, d), dtype=np.float32)
    C = rng.standard_normal((k, d), dtype=np.float32)
    if skew == "giant":
        labels = (rng.random(n) < 0.999).astype(np.int64) * 0 + (rng.random(n) < 0.001)
    elif skew == "zipf":
        labels = np.minimum(rng.zipf(1.5, size=n) - 1, k - 1).astype(np.int64)
    elif skew == "one-big":
        labels = np.where(rng.random(n) < 0.5, 7, rng.integers(0, k, size=n)).astype(np.int64)
    elif skew == "ramp":
        assert n == k * (k - 1) // 2
        labels = rng.permutation(np.repeat(np.arange(k), np.arange(k))).astype(np.int64)
    elif skew == "edge":
        assert n * d == 1 << 26 and n == 32 * k
        sizes = np.concatenate([np.arange(256), np.zeros(k - 256, dtype=np.int64)])
        rest = n - int(sizes.sum())
        sizes[256:] = rest // (k - 256)
        sizes[256:256 + rest % (k - 256)] += 1
        labels = rng.permutation(np.repeat(np.arange(k), sizes)).astype(np.int64)
    else:
        labels = rng.integers(0, k, size=n).astype(np.int64)
    C_new, counts = binding.update(gu.to_gpu(X), gu.to_gpu(labels), gu.to_gpu(C))
    torch.cuda.synchronize()
    frac = gu.check_update(X, labels, C, C_new.cpu().numpy(), counts.cpu().numpy())
    gu.announce(f"skewed update {skew}: bit-exact fraction in big clusters {frac:.6f}")
    assert frac > 0.99


@pytest.mark.parametrize("n,k,d,tile", [(1000, 37, 64, None), (4096, 32, 64, None),
                                        (65536, 256, 256, "256x256"), (1000, 37, 64, "256x256")])
def test_overflowing_centroid_norms_keep_labels_in_range(monkeypatch, n, k, d, tile):
    """Finite centroids whose float32 squared norm overflows: every candidate
    distance of a row is +inf, so the lowest index wins the +inf tie, as for
    any exact tie; labels stay in [0, k) and the update and the norms of a
    Lloyd step (fused at k >= 16 ceil(d / 256)) only ever index valid rows.
    With one finite centroid among them, that one wins every row."""
    if tile:
        monkeypatch.setenv("KMEANS_ASSIGN_TILE", tile)
    gu.announce(f"overflowing norms {n}x{k}x{d} tile {tile}")
    rng = np.random.default_rng(9)
    X = rng.standard_normal((n, d)).astype(np.float32)
    C = (np.float32(1e20) * np.sign(rng.standard_normal((k, d)))).astype(np.float32)
    assert np.square(C.astype(np.float64)).sum(axis=1).min() > np.finfo(np.float32).max
    labels, md, C_new, counts = gu.gpu_lloyd(X, C)
    assert labels.min() >= 0 and labels.max() < k
    assert np.all(labels == 0) and counts[0] == n and counts[1:].sum() == 0
    assert np.all(np.isinf(md))
    gu.check_update(X, labels, C, C_new, counts)
    C[k // 2] = X[7]
    labels, md, C_new, counts = gu.gpu_lloyd(X, C)
    assert np.all(labels == k // 2) and counts[k // 2] == n
    gu.check_update(X, labels, C, C_new, counts)
