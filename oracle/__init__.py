"""float64 brute-force CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the
benchmark may import this package. It shares no code with the GPU path; the GPU
path must never call it.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over the outer loop,
float64, difference form). This module only builds and loads that library,
marshals numpy arrays, and derives the near-tie mask from the oracle's best and
second-best distances.

Functions and the passages they follow:

* ``assign``  - squared distance in the explicit difference form and the
  lowest-index argmin ("Fusion probe", section PyTorch, naive argmin;
  "Three shapes that fit an eager Gram assignment", section Running argmin).
* ``update``  - per-cluster counts, sums and means ("Three shapes ...", section
  Full Lloyd step; "004 - tile sizes ...", section Cython reference). Empty
  clusters keep their old centre.
* ``lloyd_step`` - ``assign`` with the old centres, then ``update`` with those
  labels ("004 - tile sizes ...", section Cython reference: the assignment
  precedes the scatter into centre sums).
* ``kmeanspp`` - greedy k-means++ seeding with the random draws passed in
  ("004 - tile sizes ...", section k-means++: 2 + log(k) candidate trials per
  centre); the steps are written out in ``oracle.c``. ``default_trials`` is
  that trial count.
* ``relocate``, ``fit`` - the Lloyd driver with empty-cluster relocation
  ("004 - tile sizes ...", section Cython timing); the relocation rule is a
  reading, stated above ``relocate``.
* ``near_ties`` - rows whose best-to-second-best gap is within
  ``rtol * (||x||^2 + ||c_label||^2)``; on these rows two correct float32
  implementations may pick different labels ("004 - tile sizes ...", section
  Same arrays as the Cython iteration, where two implementations disagree on
  one row of 65536).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

_lock = threading.Lock()
_lib = None

_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")


def build(verbose: bool = False, src: str = SRC_PATH, out: str = LIB_PATH) -> str:
    """Compile ``oracle.c`` (or ``src``) into a shared library with gcc and OpenMP."""
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"expected float32, got {a.dtype}")
    return a


class Oracle:
    """The oracle bound to one compiled library (the default one unless a test
    loads a build with a planted mistake to show the pins catch it)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_assign.restype = None
        lib.oracle_assign.argtypes = [_f32p, _f32p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, _i64p, _f64p, _f64p]
        lib.oracle_update.restype = ctypes.c_int
        lib.oracle_update.argtypes = [_f32p, _i64p, _f32p, ctypes.c_int64, ctypes.c_int64,
                                      ctypes.c_int64, _f32p, _i64p, _f64p]
        i64 = ctypes.c_int64
        lib.oracle_kmeanspp.restype = None
        lib.oracle_kmeanspp.argtypes = [_f32p, i64, i64, i64, i64, i64, _f64p, _i64p, _f64p,
                                        _f64p, _i64p, _f64p]
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        """Threads the oracle's OpenMP loops use."""
        return int(self.lib.oracle_num_threads())

    def assign(self, X, C):
        """Nearest centroid of every row of X.

        Returns ``(labels, best, second)``: int64 labels (lowest index on exact
        ties), float64 D_i,label and float64 second-smallest distance over the
        other centroids (+inf if k = 1).
        """
        X, C = _f32(X), _f32(C)
        n, d = X.shape
        k, d2 = C.shape
        if d != d2:
            raise ValueError("X and C disagree on d")
        labels = np.empty(n, dtype=np.int64)
        best = np.empty(n, dtype=np.float64)
        second = np.empty(n, dtype=np.float64)
        if n:
            self.lib.oracle_assign(X, C, n, k, d, labels, best, second)
        return labels, best, second

    def update(self, X, labels, C_old):
        """Lloyd centroid update for fixed labels.

        Returns ``(C_new, counts, sums)``: float32 (k, d) means (old centre kept
        for an empty cluster), int64 counts, float64 (k, d) per-cluster sums.
        """
        X, C_old = _f32(X), _f32(C_old)
        labels = np.ascontiguousarray(labels, dtype=np.int64)
        n, d = X.shape
        k = C_old.shape[0]
        if labels.shape != (n,):
            raise ValueError("labels must have shape (n,)")
        C_new = np.empty((k, d), dtype=np.float32)
        counts = np.empty(k, dtype=np.int64)
        sums = np.empty((k, d), dtype=np.float64)
        rc = self.lib.oracle_update(X, labels, C_old, n, k, d, C_new, counts, sums)
        if rc != 0:
            raise ValueError("a label lies outside [0, k)")
        return C_new, counts, sums

    def kmeanspp(self, X, k, first, trials, rand):
        """Greedy k-means++ seeding with the given draws (see oracle.c).

        rand: (k - 1, trials) uniforms in [0, 1). Returns (chosen indices,
        final potential is not returned; centres = X[chosen]).
        """
        X = _f32(X)
        n, d = X.shape
        rand = np.ascontiguousarray(rand, dtype=np.float64).reshape(-1)
        if not (1 <= k <= n) or trials < 1 or rand.size < (k - 1) * trials:
            raise ValueError("bad k-means++ arguments")
        chosen = np.empty(k, dtype=np.int64)
        closest = np.empty(n, dtype=np.float64)
        cand_d = np.empty(max(trials * n, 1), dtype=np.float64)
        cand = np.empty(trials, dtype=np.int64)
        pots = np.empty(trials, dtype=np.float64)
        if rand.size == 0:
            rand = np.zeros(1, dtype=np.float64)
        self.lib.oracle_kmeanspp(X, n, d, k, int(first), trials, rand, chosen, closest, cand_d,
                                 cand, pots)
        return chosen

    def lloyd_step(self, X, C_old):
        """One Lloyd iteration: labels against C_old, then the mean update.

        Returns ``(labels, best, second, C_new, counts)``.
        """
        labels, best, second = self.assign(X, C_old)
        C_new, counts, _ = self.update(X, labels, C_old)
        return labels, best, second, C_new, counts


def default() -> Oracle:
    """The oracle built from ``oracle.c`` (built on first use if missing)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                build()
            _lib = Oracle(LIB_PATH)
        return _lib


def num_threads() -> int:
    return default().num_threads()


def assign(X, C):
    return default().assign(X, C)


def update(X, labels, C_old):
    return default().update(X, labels, C_old)


def lloyd_step(X, C_old):
    return default().lloyd_step(X, C_old)


def kmeanspp(X, k, first, trials, rand):
    return default().kmeanspp(X, k, first, trials, rand)


def default_trials(k: int) -> int:
    """The pages' trial count 2 + log(k) ("004 - tile sizes ...", section
    k-means++), read as the natural logarithm truncated to an integer:
    2 + floor(ln k), e.g. 8 at k = 1024 and 2 at k = 1."""
    import math

    return 2 + int(math.log(k)) if k > 0 else 2


def sq_norms(A, rows_per_chunk: int = 4096) -> np.ndarray:
    """Row squared norms, every element widened to float64 (a chunk of rows
    at a time, so a large float32 matrix is never copied whole)."""
    A = np.asarray(A)
    out = np.empty(A.shape[0], dtype=np.float64)
    for r0 in range(0, A.shape[0], rows_per_chunk):
        A64 = A[r0:r0 + rows_per_chunk].astype(np.float64)
        out[r0:r0 + rows_per_chunk] = np.einsum("ij,ij->i", A64, A64)
    return out


def tie_band(X, C, labels, rtol: float = 1e-5) -> np.ndarray:
    """Width of the near-tie band of every row: rtol * (||x_i||^2 +
    ||c_label_i||^2), norms in float64, c the row's oracle winner."""
    return rtol * (sq_norms(X) + sq_norms(C)[np.asarray(labels)])


def near_ties(X, C, labels, best, second, rtol: float = 1e-5) -> np.ndarray:
    """Boolean mask of rows whose best-to-second gap is within the tie band:
    second - best <= rtol * (||x_i||^2 + ||c_label_i||^2) (``tie_band``)."""
    return (np.asarray(second) - np.asarray(best)) <= tie_band(X, C, labels, rtol)


for _name in ("num_threads", "assign", "update", "lloyd_step", "kmeanspp"):
    globals()[_name].__doc__ = getattr(Oracle, _name).__doc__
del _name


# --------------------------------------------------------------------------
# Lloyd driver with empty-cluster relocation ("004 - tile sizes ...", section
# Cython timing: the Lloyd call updates the centres and relocates empty
# clusters). The pages do not give the relocation rule; the reading used here:
#
#   after the assignment against the old centres, let E be the empty clusters
#   in increasing index and m = min(|E|, n). The m samples farthest from their
#   assigned old centre (float64 difference-form distance, larger first, lower
#   sample index first on equal distances) are moved, the r-th of them becoming
#   the only member of cluster E[r]. The update then runs on the new labels; a
#   cluster emptied by a move keeps its old centre.
#
# The driver repeats assignment (+ relocation) + update from C_init until the
# centre shift sum_j ||C_new_j - C_old_j||^2 (float64) is <= tol or max_iter
# iterations ran, then assigns once more against the final centres; inertia is
# the sum of those final squared distances.


def relocate(labels, best, k):
    """Apply the relocation rule above; returns (new_labels, moves) where
    moves is a list of (sample, new_cluster) pairs in order."""
    labels = np.array(labels, dtype=np.int64, copy=True)
    n = len(labels)
    counts = np.bincount(labels, minlength=k)
    empty = np.nonzero(counts == 0)[0]
    m = min(len(empty), n)
    if m == 0:
        return labels, []
    order = np.lexsort((np.arange(n), -np.asarray(best, dtype=np.float64)))
    moves = [(int(order[r]), int(empty[r])) for r in range(m)]
    for i, j in moves:
        labels[i] = j
    return labels, moves


def centre_shift(C_new, C_old) -> float:
    """sum_j ||C_new_j - C_old_j||^2 in float64."""
    diff = np.asarray(C_new, dtype=np.float64) - np.asarray(C_old, dtype=np.float64)
    return float(np.sum(diff * diff))


def fit(X, C_init, max_iter: int, tol: float, relocate_empty: bool):
    """Lloyd iterations from C_init (see the rule above).

    Returns a dict: labels, best (final squared distances), centres, counts,
    n_iter, inertia, shift (the last iteration's centre shift), history (the
    centre shift of every iteration).
    """
    orc = default()
    C = np.array(C_init, dtype=np.float32, copy=True)
    k = C.shape[0]
    history = []
    n_iter = 0
    shift = 0.0
    for it in range(max_iter):
        labels, best, _ = orc.assign(X, C)
        if relocate_empty:
            labels, _ = relocate(labels, best, k)
        C_new, _, _ = orc.update(X, labels, C)
        shift = centre_shift(C_new, C)
        history.append(shift)
        C = C_new
        n_iter = it + 1
        if shift <= tol:
            break
    labels, best, _ = orc.assign(X, C)
    counts = np.bincount(labels, minlength=k).astype(np.int64)
    return {"labels": labels, "best": best, "centres": C, "counts": counts,
            "n_iter": n_iter, "inertia": float(np.sum(best)), "shift": shift,
            "history": history}
