"""Each plausible slip planted in a copy of the oracle fails at least one pin.

The copies are built on the CPU into a temporary directory; the real oracle
source is never modified.
"""
import os
import tempfile

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
