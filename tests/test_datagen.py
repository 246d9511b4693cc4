"""The seeded input generators (no GPU)."""
import numpy as np

from nearest_centroid_assignment_amd import datagen


def test_same_seed_same_bytes():
    a = datagen.make("probe", seed=0)
    b = datagen.make("probe", seed=0)
    c = datagen.make("probe", seed=1)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not np.array_equal(a[0], c[0])


def test_shapes_dtypes_and_distinct_rows():
    for name in ("tiny", "probe"):
        cfg = datagen.CONFIGS[name]
        X, C = datagen.make(name)
        assert X.shape == (cfg.n, cfg.d) and C.shape == (cfg.k, cfg.d)
        assert X.dtype == np.float32 and C.dtype == np.float32
        assert X.flags.c_contiguous and C.flags.c_contiguous
        # C is made of distinct rows of X
        assert len(np.unique(C, axis=0)) == cfg.k
        rows = {r.tobytes() for r in X}
        assert all(r.tobytes() in rows for r in C)


def test_blob_statistics():
    """Tiny: 17 blobs with centre spread 4 and unit noise."""
    X, _ = datagen.make("tiny")
    cfg = datagen.CONFIGS["tiny"]
    assert abs(X.std() - np.sqrt(cfg.sigma_c**2 + cfg.sigma**2)) < 0.3


def test_block_streams_independent_of_threads(monkeypatch):
    """The parallel block fill gives the same bytes as a serial fill."""
    out1 = np.empty((10000, 3), dtype=np.float32)
    datagen._fill_normal(5, 2, out1, block_rows=777)
    monkeypatch.setattr(datagen.os, "cpu_count", lambda: 1)
    out2 = np.empty((10000, 3), dtype=np.float32)
    datagen._fill_normal(5, 2, out2, block_rows=777)
    assert np.array_equal(out1, out2)
    ref = np.random.default_rng([5, 2, 1]).standard_normal((777, 3), dtype=np.float32)
    assert np.array_equal(out1[777:1554], ref)


def test_integer_and_far_centroid():
    X, C = datagen.make_integer(50, 5, 7)
    assert np.all(X == np.round(X)) and np.abs(X).max() <= 8
    C2 = datagen.with_far_centroid(X, C, 2)
    assert np.all(C2[2] > np.abs(X).max())
    assert np.array_equal(np.delete(C2, 2, 0), np.delete(C, 2, 0))
