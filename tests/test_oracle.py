"""The float64 oracle against its pins (no GPU)."""
import numpy as np
import pytest

from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(oracle_mod, pin):
    pin(oracle_mod.default())


def test_round_to_f32_helper():
    """The rational rounding helper used by the update pin: ties go to even."""
    from fractions import Fraction

    one = np.float32(1.0)
    ulp = Fraction(float(np.nextafter(one, np.float32(2))) - 1.0)
    assert pins.round_to_f32(Fraction(1) + ulp / 2) == one  # tie -> even (1.0)
    up = np.nextafter(one, np.float32(2))
    assert pins.round_to_f32(Fraction(1) + 3 * ulp / 2) == np.nextafter(up, np.float32(2))
    assert pins.round_to_f32(Fraction(1, 3)) == np.float32(1 / 3)


def test_near_tie_band(oracle_mod):
    """A duplicated centroid is an exact tie: gap 0, inside the band."""
    X = np.array([[0.0, 1.0], [5.0, 5.0]], dtype=np.float32)
    C = np.array([[0.0, 0.0], [0.0, 0.0], [9.0, 9.0]], dtype=np.float32)
    labels, best, second = oracle_mod.assign(X, C)
    ties = oracle_mod.near_ties(X, C, labels, best, second)
    assert labels.tolist() == [0, 2]  # (5,5): 50 to the origin, 32 to (9,9)
    assert ties.tolist() == [True, False]


def test_second_formulation_small_configs(oracle_mod):
    """numpy float64 Gram + first-occurrence argmin agrees with the oracle on
    the Tiny and Probe workloads on every row outside the near-tie band (Tiny
    has none; Probe has one)."""
    from nearest_centroid_assignment_amd import datagen

    for name, max_ties in (("tiny", 0), ("probe", 1)):
        X, C = datagen.make(name)
        labels, best, second = oracle_mod.assign(X, C)
        X64, C64 = X.astype(np.float64), C.astype(np.float64)
        G = (C64 * C64).sum(1)[None, :] - 2.0 * X64 @ C64.T
        ties = oracle_mod.near_ties(X, C, labels, best, second)
        assert ties.sum() <= max_ties
        assert np.array_equal(np.argmin(G, axis=1)[~ties], labels[~ties])


def test_thread_count_independent(oracle_mod, monkeypatch):
    """Results do not depend on how OpenMP splits the outer loop."""
    from nearest_centroid_assignment_amd import datagen

    X, C = datagen.make("probe")
    ref = oracle_mod.lloyd_step(X, C)
    import subprocess, sys, os, json

    code = (
        "import sys, numpy as np; sys.path.insert(0, %r);"
        "import oracle; from nearest_centroid_assignment_amd import datagen;"
        "X, C = datagen.make('probe'); l, b, s, Cn, cnt = oracle.lloyd_step(X, C);"
        "np.save(sys.argv[1], np.concatenate([l.astype(np.float64), b, s, Cn.ravel().astype(np.float64)]))"
        % os.getcwd()
    )
    import tempfile

    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "r.npy")
        env = dict(os.environ, OMP_NUM_THREADS="3")
        subprocess.run([sys.executable, "-c", code, out], check=True, env=env,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
        got = np.load(out)
    want = np.concatenate([ref[0].astype(np.float64), ref[1], ref[2], ref[3].ravel().astype(np.float64)])
    assert np.array_equal(got, want)
