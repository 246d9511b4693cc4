"""Each plausible slip planted in a copy of the oracle fails at least one pin.

The copies of the C library are built on the CPU into a temporary directory;
the real oracle source is never modified. The Python helpers are replaced, one
at a time, in a namespace that otherwise forwards to the real oracle module.
"""
import math
import os
import tempfile
import types

import numpy as np

import pytest

import oracle
from tests import oracle_pins as pins

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("tie_to_highest_index", "if (s < b1) {", "if (s <= b1) {"),
    ("wrong_sign", "(double)x[t] - (double)c[t]", "(double)x[t] + (double)c[t]"),
    ("dropped_square", "double diff = (double)x[t] - (double)c[t];\n                s += diff * diff;",
     "double diff = (double)x[t] - (double)c[t];\n                s += diff;"),
    ("centroid_row_index", "const float *c = C + j * d;", "const float *c = C + j;"),
    ("sample_row_index", "const float *x = X + i * d;\n        double b1", "const float *x = X + i;\n        double b1"),
    ("dropped_last_term", "for (int64_t t = 0; t < d; ++t) {\n                double diff",
     "for (int64_t t = 0; t < d - 1; ++t) {\n                double diff"),
    ("second_not_demoted", "b2 = b1;\n                b1 = s;", "b1 = s;"),
    ("second_misses_later", "} else if (s < b2) {", "} else if (s < b2 && 0) {"),
    ("count_not_accumulated", "counts[labels[i]] += 1;", "counts[labels[i]] = 1;"),
    ("mean_off_by_one", "sums[j * d + t] / (double)counts[j]", "sums[j * d + t] / (double)(counts[j] + 1)"),
    ("empty_cluster_zeroed", "C_new[j * d + t] = C_old[j * d + t];", "C_new[j * d + t] = 0.0f;"),
    ("update_transposed", "const float *x = X + i * d;\n            double *s", "const float *x = X + i;\n            double *s"),
    ("sum_in_float", "s[t] += (double)x[t];", "s[t] = (float)(s[t] + x[t]);"),
    ("pp_search_strict", "if (acc >= target) {", "if (acc > target + 1.0) {"),
    ("pp_highest_potential", "if (pots[t] < pots[best]) best = t;", "if (pots[t] > pots[best]) best = t;"),
    ("pp_no_min", "dt[i] = di < closest[i] ? di : closest[i];", "dt[i] = di;"),
    ("pp_stale_pot", "pot = pots[best];", "pot = pot;"),
    ("pp_wrong_row", "const float *x = X + a * d, *y = X + b * d;", "const float *x = X + a * d, *y = X + b;"),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC_PATH) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(source, name, old, new):
    assert source.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    with tempfile.TemporaryDirectory() as tmp:
        src = os.path.join(tmp, f"{name}.c")
        with open(src, "w") as f:
            f.write(source.replace(old, new))
        lib = oracle.build(src=src, out=os.path.join(tmp, f"{name}.so"))
        orc = oracle.Oracle(lib)
        caught = []
        for pin in pins.ALL_PINS:
            try:
                pin(orc)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin catches the planted mistake {name}"


def _ns(**override):
    """The oracle module's helpers, with some replaced."""
    ns = types.SimpleNamespace(centre_shift=oracle.centre_shift, near_ties=oracle.near_ties,
                               default_trials=oracle.default_trials)
    for k, v in override.items():
        setattr(ns, k, v)
    return ns


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def _ties_with_scale(scale_fn):
    def near_ties(X, C, labels, best, second, rtol=1e-5):
        return (_f64(second) - _f64(best)) <= rtol * scale_fn(X, C, labels, best, second)
    return near_ties


def _n(A):
    return oracle.sq_norms(A)


PY_MUTANTS = [
    ("shift_dropped_square", "centre_shift",
     lambda a, b: float(np.sum(_f64(a) - _f64(b)))),
    ("shift_abs_not_square", "centre_shift",
     lambda a, b: float(np.sum(np.abs(_f64(a) - _f64(b))))),
    ("shift_sqrt_per_centre", "centre_shift",
     lambda a, b: float(np.sum(np.sqrt(((_f64(a) - _f64(b)) ** 2).sum(1))))),
    ("shift_max_not_sum", "centre_shift",
     lambda a, b: float(np.max(((_f64(a) - _f64(b)) ** 2).sum(1)))),
    ("shift_in_float32", "centre_shift",
     lambda a, b: float(np.sum((np.asarray(a, np.float32) - np.asarray(b, np.float32)) ** 2,
                               dtype=np.float32))),
    ("ties_dropped_x_norm", "near_ties",
     _ties_with_scale(lambda X, C, l, b, s: _n(C)[np.asarray(l)])),
    ("ties_runner_up_norm", "near_ties",
     # the norm of the centroid that is not the winner (k = 2 in the pins)
     _ties_with_scale(lambda X, C, l, b, s: _n(X) + _n(C)[(np.asarray(l) + 1) % len(C)])),
    ("ties_max_centroid_norm", "near_ties",
     _ties_with_scale(lambda X, C, l, b, s: _n(X) + _n(C).max())),
    ("ties_relative_to_best", "near_ties",
     _ties_with_scale(lambda X, C, l, b, s: _f64(b))),
    ("ties_strict", "near_ties",
     lambda X, C, l, b, s, rtol=1e-5: (_f64(s) - _f64(b)) < oracle.tie_band(X, C, l, rtol)),
    ("trials_log2", "default_trials", lambda k: 2 + int(math.log2(k))),
    ("trials_log10", "default_trials", lambda k: 2 + int(math.log10(k))),
    ("trials_rounded", "default_trials", lambda k: 2 + round(math.log(k))),
    ("trials_ceil", "default_trials", lambda k: 2 + math.ceil(math.log(k))),
    ("trials_no_two", "default_trials", lambda k: int(math.log(k))),
]


@pytest.mark.parametrize("name,helper,fn", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_python_mutant_is_caught(name, helper, fn):
    ns = _ns(**{helper: fn})
    caught = []
    for pin in pins.PY_PINS:
        try:
            pin(ns, oracle.default())
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
