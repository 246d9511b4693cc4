"""Pins for the float64 oracle: checks against facts fixed by mathematics, not by
the oracle itself.

Each ``pin_*`` function takes an oracle object (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees with the fact it checks. The same
functions run on the real oracle (tests/test_oracle.py) and on builds of it with
a planted mistake (tests/test_oracle_mutants.py), which shows that a plausible
slip anywhere in the oracle fails at least one pin.

What pins what:

* ``pin_exhaustive_small``  - every labelling of tiny integer problems is
  enumerated with exact integer arithmetic. The total squared error is separable
  over rows, so the set of minimisers is the product of per-row argmin sets and
  its lexicographically first element is the per-row lowest-index argmin. This
  fixes the distance, the argmin, the lowest-index tie rule and the
  second-best distance.
* ``pin_exhaustive_grid``   - all X in {0,1,2}^3 (d = 1) against all C in
  {0,1,2}^2: every small tie pattern.
* ``pin_update_exact``      - for fixed labels the new centre is the exact
  rational mean (Fraction), rounded once to float32 (round to nearest, ties to
  even); an empty cluster keeps its old centre.
* ``pin_gram_identity``     - the Gram expansion ||x||^2 + ||c||^2 - 2 x.c
  ("Three shapes that fit an eager Gram assignment", section Gram assignment)
  equals the oracle's difference form, and dropping ||x||^2 ("004 - tile
  sizes ...", section Schedules added) leaves the argmin unchanged.
* ``pin_invariants``        - translation invariance, centroid permutation,
  k = 1, C = X, duplicate centroids, Lloyd monotonicity.
* ``pin_kmeanspp_*``        - k-means++ seeding ("004 - tile sizes ...", section
  k-means++): a hand-worked draw; with one trial, over evenly spaced draws each
  sample is taken for a fraction D(i)/pot of them (D^2 sampling); each centre
  is the trial candidate of least potential (recomputed with numpy) and the
  potential never rises.
"""
from __future__ import annotations

import itertools
from fractions import Fraction

import numpy as np

# ---------------------------------------------------------------- helpers


def exact_sq_dist(x, c) -> int:
    """Squared distance of two integer-valued vectors, in Python integers."""
    return sum((int(a) - int(b)) ** 2 for a, b in zip(x, c))


def round_to_f32(q: Fraction) -> np.float32:
    """Round a rational number to the nearest float32, ties to even mantissa.

    Built from the definition: take the float32 nearest to float(q) and its two
    neighbours, and keep the candidate at the smallest exact distance from q.
    """
    f = np.float32(float(q))
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    best = None
    for c in cands:
        err = abs(Fraction(float(c)) - q)
        key = (err, int(np.frombuffer(np.float32(c).tobytes(), dtype=np.uint32)[0]) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def f32_bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def brute_labelling(X, C):
    """Enumerate all labellings; return (lexicographically first minimiser,
    per-row exact best, per-row exact second best or None)."""
    n, k = len(X), len(C)
    D = [[exact_sq_dist(X[i], C[j]) for j in range(k)] for i in range(n)]
    best_total, best_lab = None, None
    for lab in itertools.product(range(k), repeat=n):
        total = sum(D[i][lab[i]] for i in range(n))
        if best_total is None or total < best_total:
            best_total, best_lab = total, lab
    best = [D[i][best_lab[i]] for i in range(n)]
    second = []
    for i in range(n):
        others = [D[i][j] for j in range(k) if j != best_lab[i]]
        second.append(min(others) if others else None)
    return list(best_lab), best, second


def _check_against_brute(orc, X, C):
    labels, best, second = orc.assign(X, C)
    lab_ref, best_ref, second_ref = brute_labelling(X.tolist(), C.tolist())
    assert labels.tolist() == lab_ref, (labels.tolist(), lab_ref, X.tolist(), C.tolist())
    assert best.tolist() == [float(v) for v in best_ref]
    for s, r in zip(second.tolist(), second_ref):
        if r is None:
            assert s == float("inf")
        else:
            assert s == float(r)


# ------------------------------------------------------------------- pins


def pin_exhaustive_small(orc, cases: int = 60, seed: int = 1):
    rng = np.random.default_rng(seed)
    for case in range(cases):
        n = int(rng.integers(1, 7))
        k = int(rng.integers(1, 4))
        d = int(rng.integers(1, 4))
        X = rng.integers(-2, 3, size=(n, d)).astype(np.float32)
        C = rng.integers(-2, 3, size=(k, d)).astype(np.float32)
        if k >= 2 and case % 3 == 0:
            C[k - 1] = C[0]  # a duplicate centroid: the lower index must win
        _check_against_brute(orc, X, C)


def pin_exhaustive_grid(orc):
    for xs in itertools.product(range(3), repeat=3):
        X = np.array(xs, dtype=np.float32).reshape(3, 1)
        for cs in itertools.product(range(3), repeat=2):
            C = np.array(cs, dtype=np.float32).reshape(2, 1)
            _check_against_brute(orc, X, C)


def pin_update_exact(orc, seed: int = 2):
    rng = np.random.default_rng(seed)
    for trial in range(6):
        n, k, d = 40 + 7 * trial, 9, 5
        if trial % 2 == 0:
            X = rng.integers(-8, 9, size=(n, d)).astype(np.float32)
        else:
            X = rng.standard_normal((n, d), dtype=np.float32)
        labels = rng.integers(0, k - 2, size=n).astype(np.int64)  # k-2, k-1 stay empty
        labels[0] = 0
        C_old = rng.standard_normal((k, d), dtype=np.float32)
        C_new, counts, sums = orc.update(X, labels, C_old)
        for j in range(k):
            rows = [i for i in range(n) if labels[i] == j]
            assert counts[j] == len(rows)
            for t in range(d):
                exact = sum((Fraction(float(X[i, t])) for i in rows), Fraction(0))
                assert Fraction(float(sums[j, t])) == exact
                if rows:
                    want = round_to_f32(exact / len(rows))
                else:
                    want = C_old[j, t]
                assert f32_bits(C_new[j, t]) == f32_bits(want), (j, t, C_new[j, t], want)


def _blobs(n, k, d, seed):
    rng = np.random.default_rng(seed)
    centres = 3.0 * rng.standard_normal((k, d))
    X = (centres[rng.integers(0, k, size=n)] + rng.standard_normal((n, d))).astype(np.float32)
    C = X[rng.choice(n, k, replace=False)].copy()
    return X, C


def pin_gram_identity(orc, seed: int = 3):
    X, C = _blobs(300, 23, 37, seed)
    labels, best, second = orc.assign(X, C)
    X64, C64 = X.astype(np.float64), C.astype(np.float64)
    xn = (X64 * X64).sum(1)
    cn = (C64 * C64).sum(1)
    G = xn[:, None] + cn[None, :] - 2.0 * (X64 @ C64.T)
    rows = np.arange(len(X))
    scale = xn + cn[labels]
    assert np.all(np.abs(G[rows, labels] - best) <= 1e-12 * scale + 1e-300)
    Gs = np.sort(G, axis=1)
    gap = Gs[:, 1] - Gs[:, 0]
    clear = gap > 1e-9 * (xn + cn.max())
    assert clear.mean() > 0.9
    assert np.array_equal(np.argmin(G, axis=1)[clear], labels[clear])
    # Dropping ||x||^2 leaves the argmin unchanged.
    Gd = cn[None, :] - 2.0 * (X64 @ C64.T)
    assert np.array_equal(np.argmin(Gd, axis=1)[clear], labels[clear])
    # The second-best distance is the second order statistic of the row.
    assert np.all(np.abs(Gs[:, 1] - second) <= 1e-12 * (xn + cn.max()))


def pin_invariants(orc, seed: int = 4):
    rng = np.random.default_rng(seed)
    # Translation by an integer vector keeps integer data exact in float32.
    X = rng.integers(-8, 9, size=(64, 6)).astype(np.float32)
    C = rng.integers(-8, 9, size=(7, 6)).astype(np.float32)
    v = rng.integers(-50, 51, size=6).astype(np.float32)
    l0, b0, s0 = orc.assign(X, C)
    l1, b1, s1 = orc.assign(X + v, C + v)
    assert np.array_equal(l0, l1) and np.array_equal(b0, b1) and np.array_equal(s0, s1)

    # Permuting centroids permutes the labels (data without near ties).
    Xb, Cb = _blobs(200, 11, 9, seed + 1)
    lb, bb, sb = orc.assign(Xb, Cb)
    perm = rng.permutation(len(Cb))
    lp, bp, _ = orc.assign(Xb, Cb[perm])
    inv = np.argsort(perm)
    assert np.array_equal(inv[lb], lp)
    assert np.allclose(bb, bp, rtol=1e-13, atol=0)

    # k = 1: every label is 0 and the new centre is the column mean.
    l1c, _, s1c = orc.assign(Xb, Cb[:1])
    assert np.all(l1c == 0) and np.all(np.isinf(s1c))
    Cn, cnt, _ = orc.update(Xb, l1c, Cb[:1])
    assert cnt.tolist() == [len(Xb)]
    assert np.allclose(Cn[0], Xb.astype(np.float64).mean(0), rtol=1e-6, atol=1e-6)

    # C = X with distinct rows: sample i is its own centroid, at distance 0.
    Xs = Xb[:40]
    ls, bs, _ = orc.assign(Xs, Xs)
    assert np.array_equal(ls, np.arange(40)) and np.all(bs == 0.0)

    # Duplicate centroid rows: the lower index wins, the higher never does.
    Cd = np.concatenate([Cb, Cb[3:4]], axis=0)
    ld, _, sd = orc.assign(Xb, Cd)
    assert not np.any(ld == len(Cb))
    assert np.all(sd[ld == 3] == bb[ld == 3])

    # Lloyd monotonicity: the update never raises the within-cluster error.
    Xm, Cm = _blobs(500, 9, 8, seed + 2)
    for _ in range(3):
        lm, bm, _ = orc.assign(Xm, Cm)
        Cn, _, _ = orc.update(Xm, lm, Cm)
        _, bn, _ = orc.assign(Xm, Cn)
        assert bn.sum() <= bm.sum() * (1 + 1e-9)
        Cm = Cn


ALL_PINS = [pin_exhaustive_small, pin_exhaustive_grid, pin_update_exact,
            pin_gram_identity, pin_invariants]


# ------------------------------------------------------------------ k-means++


def _dist64(X, a, b):
    diff = X[a].astype(np.float64) - X[b].astype(np.float64)
    return float(diff @ diff)


def pin_kmeanspp_hand(orc):
    """1-D samples 0, 1, 3 with the first centre at 0: D = 0, 1, 9, pot = 10.
    u = 0.05 -> target 0.5 -> sample 1 (running sums 0, 1, 10); u = 0.5 ->
    target 5 -> sample 2. Worked by hand from the definition."""
    X = np.array([[0], [1], [3]], dtype=np.float32)
    assert orc.kmeanspp(X, 2, 0, 1, np.array([[0.05]])).tolist() == [0, 1]
    assert orc.kmeanspp(X, 2, 0, 1, np.array([[0.5]])).tolist() == [0, 2]
    # Two trials: candidates 1 and 2; potentials min(D, d(., 1)) = 0+0+4 = 4 and
    # min(D, d(., 2)) = 0+1+0 = 1, so the second wins.
    assert orc.kmeanspp(X, 2, 0, 2, np.array([[0.05, 0.5]])).tolist() == [0, 2]


def pin_kmeanspp_d2_quadrature(orc, seed: int = 6):
    """With one trial, D^2 sampling: over u = (j + 1/2) / N the second centre is
    sample i for a fraction D(i) / pot of the draws (to within 1/N each)."""
    rng = np.random.default_rng(seed)
    X = rng.integers(-5, 6, size=(9, 2)).astype(np.float32)
    first = 4
    D = np.array([_dist64(X, i, first) for i in range(len(X))])
    N = 2000
    hits = np.zeros(len(X))
    for j in range(N):
        c = orc.kmeanspp(X, 2, first, 1, np.array([[(j + 0.5) / N]]))
        hits[c[1]] += 1
    assert np.all(np.abs(hits / N - D / D.sum()) <= 1.0 / N + 1e-12)


def pin_kmeanspp_greedy(orc, seed: int = 7):
    """Each chosen centre is, among its trials' candidates (recomputed here
    from the same draws with numpy), the one of smallest potential, and the
    potential never rises."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((300, 5)).astype(np.float32)
    k, trials = 12, 4
    u = rng.random((k - 1, trials))
    chosen = orc.kmeanspp(X, k, 17, trials, u)
    X64 = X.astype(np.float64)
    D = ((X64 - X64[17]) ** 2).sum(1)
    assert chosen[0] == 17
    prev_pot = D.sum()
    for c in range(1, k):
        cum = np.cumsum(D)
        cands = [min(int(np.searchsorted(cum, u[c - 1, t] * D.sum(), side="left")), len(X) - 1)
                 for t in range(trials)]
        pots = [np.minimum(D, ((X64 - X64[i]) ** 2).sum(1)).sum() for i in cands]
        best = int(np.argmin(pots))
        assert chosen[c] == cands[best]
        D = np.minimum(D, ((X64 - X64[chosen[c]]) ** 2).sum(1))
        assert D.sum() <= prev_pot
        prev_pot = D.sum()
    assert len(set(chosen.tolist())) == k  # distinct points give distinct centres


ALL_PINS += [pin_kmeanspp_hand, pin_kmeanspp_d2_quadrature, pin_kmeanspp_greedy]


# ------------------------------------------------- the oracle's Python helpers
#
# centre_shift, near_ties and default_trials live in oracle/__init__.py, not
# in the C library. Their pins take a namespace holding the helper under test
# (the oracle module itself, or a copy with one helper replaced by a planted
# mistake in tests/test_oracle_mutants.py) and an Oracle for the assignment.


def pin_centre_shift(ns, orc):
    """The driver's convergence measure sum_j ||C_new_j - C_old_j||^2 in
    float64. The pages time fixed iteration counts ("004 - tile sizes ...",
    section Cython timing); the stopping test on the squared centre movement
    summed over centres is the reading the driver takes."""
    # Worked by hand: moves (3, 4), (0, 1) and (0, 0) -> 25 + 1 + 0 = 26.
    C_old = np.array([[0, 0], [1, 1], [2, -3]], dtype=np.float32)
    C_new = np.array([[3, 4], [1, 2], [2, -3]], dtype=np.float32)
    assert ns.centre_shift(C_new, C_old) == 26.0
    assert ns.centre_shift(C_old, C_new) == 26.0  # symmetric in its arguments
    # A common translation v moves every centre by ||v||^2: k * ||v||^2.
    rng = np.random.default_rng(12)
    C = rng.integers(-50, 51, size=(7, 5)).astype(np.float32)
    v = np.array([1, -2, 3, 0, 5], dtype=np.float32)
    assert ns.centre_shift(C + v, C) == 7.0 * float(v.astype(np.int64) @ v.astype(np.int64))
    # 4097^2 = 16785409 has no float32 representation (it needs 25 bits):
    # the squares and the sum are float64.
    assert ns.centre_shift(np.array([[4097.0]], np.float32), np.zeros((1, 1), np.float32)) \
        == 16785409.0


def pin_near_tie_band(ns, orc):
    """The band of the parity rule: a row is a near tie when its gap between
    the best and the second-best distance is <= 1e-5 * (||x||^2 + ||c||^2),
    c the winning centroid, norms in float64 ("004 - tile sizes ...", section
    Same arrays as the Cython iteration, for why such rows may differ)."""
    # Gap exactly on the band: x = (100, 200, 0) is itself centroid 0 (D = 0)
    # and centroid 1 is one unit away (D = 1); ||x||^2 + ||c_0||^2 = 100000,
    # band = 1e-5 * 100000 = 1 (exactly, in float64) = the gap: a tie.
    assert 1e-5 * 100000.0 == 1.0
    X = np.array([[100, 200, 0]], dtype=np.float32)
    C = np.array([[100, 200, 0], [101, 200, 0]], dtype=np.float32)
    labels, best, second = orc.assign(X, C)
    assert labels.tolist() == [0] and best.tolist() == [0.0] and second.tolist() == [1.0]
    assert ns.near_ties(X, C, labels, best, second).tolist() == [True]
    # Gap just outside the band, and only the winner's norm says so:
    # x = (150, 163, 30), ||x||^2 = 49969; c_0 = (150, 163, 31), D = 1,
    # ||c_0||^2 = 50030; c_1 = (150, 164, 29), D = 2, ||c_1||^2 = 50237.
    # Gap 1 > 1e-5 * 99999 = 0.99999: not a tie (with c_1's norm the band
    # would be 1.00206 and the row would count as one).
    X = np.array([[150, 163, 30]], dtype=np.float32)
    C = np.array([[150, 163, 31], [150, 164, 29]], dtype=np.float32)
    labels, best, second = orc.assign(X, C)
    assert labels.tolist() == [0] and best.tolist() == [1.0] and second.tolist() == [2.0]
    assert ns.near_ties(X, C, labels, best, second).tolist() == [False]
    # Same geometry seen from the other side: a far second centroid is never
    # a tie, an exact duplicate always is.
    X = np.array([[0.0, 1.0], [5.0, 5.0]], dtype=np.float32)
    C = np.array([[0.0, 0.0], [0.0, 0.0], [9.0, 9.0]], dtype=np.float32)
    labels, best, second = orc.assign(X, C)
    assert ns.near_ties(X, C, labels, best, second).tolist() == [True, False]


def pin_default_trials(ns, orc):
    """k-means++ trials per centre: 2 + log(k) ("004 - tile sizes ...",
    section k-means++), read as 2 + floor(ln k). Values from the definition:
    ln 2 = 0.69, ln 3 = 1.10, ln 7 = 1.95, ln 8 = 2.08, ln 20 = 3.00 (just
    below 3), ln 21 = 3.04, ln 1024 = 6.93."""
    table = {1: 2, 2: 2, 3: 3, 7: 3, 8: 4, 20: 4, 21: 5, 1024: 8}
    assert {k: ns.default_trials(k) for k in table} == table


PY_PINS = [pin_centre_shift, pin_near_tie_band, pin_default_trials]
