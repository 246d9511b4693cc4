"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the float64 oracle under the parity rules.

Parity rules (all checked, none relaxed):

* labels  - equal to the oracle's, except on rows whose oracle gap between the
  best and second-best distance is <= 1e-5 * (||x||^2 + ||c_label||^2) (a
  near tie). Every mismatch must be such a row, and the GPU's centroid must be
  within that band of the oracle's best distance.
* counts  - bit-exact against the oracle's update applied to the GPU's labels;
  against the oracle's own labels they may differ only by the moved rows.
* centroids - the oracle's update on the GPU's labels: per row,
  max |dC| <= 1e-4 * max |C_ref|. Clusters of at most 64 rows (128 once X
  has 2^26 elements or more and n >= 32 k) are summed in increasing sample order in float64
  on both sides, so those rows must also be bit-exact; bigger clusters add
  sixteen row parts (a different order).
* min_dist - |dD| <= 1e-4 * D_ref or |dD| <= 1e-5 * (||x||^2 + ||c||^2), D_ref
  the float64 distance to the GPU's chosen centroid.
"""
from __future__ import annotations

import sys

import numpy as np

import oracle

TIE_RTOL = 1e-5
REL_TOL = 1e-4


def announce(msg: str) -> None:
    """Print a progress line that bypasses pytest's capture (flushed now)."""
    sys.__stderr__.write(f"[gpu-test] {msg}\n")
    sys.__stderr__.flush()


def to_gpu(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def gpu_lloyd(X, C, min_dist=True):
    """One Lloyd iteration on the GPU; returns numpy (labels, md, C_new, counts)."""
    import torch

    from nearest_centroid_assignment_amd import binding

    Xg, Cg = to_gpu(X), to_gpu(C)
    labels, md, C_new, counts = binding.lloyd_step(Xg, Cg, min_dist=min_dist)
    torch.cuda.synchronize()
    return (labels.cpu().numpy(), None if md is None else md.cpu().numpy(),
            C_new.cpu().numpy(), counts.cpu().numpy())


def gpu_assign(X, C, min_dist=True):
    import torch

    from nearest_centroid_assignment_amd import binding

    labels, md = binding.assign(to_gpu(X), to_gpu(C), min_dist=min_dist)
    torch.cuda.synchronize()
    return labels.cpu().numpy(), None if md is None else md.cpu().numpy()


def sq_norms(A):
    return oracle.sq_norms(A)


def exact_dist(X, C, rows, cols, rows_per_chunk: int = 4096):
    """float64 difference-form distance of X[rows[i]] to C[cols[i]] (a chunk
    of rows at a time, so no (n, d) float64 copy of a large X is made)."""
    rows, cols = np.asarray(rows), np.asarray(cols)
    out = np.empty(len(rows), dtype=np.float64)
    for r0 in range(0, len(rows), rows_per_chunk):
        sl = slice(r0, r0 + rows_per_chunk)
        diff = X[rows[sl]].astype(np.float64) - C[cols[sl]].astype(np.float64)
        out[sl] = np.einsum("ij,ij->i", diff, diff)
    return out


def _rows_of(X, rows):
    return X if rows is None else X[rows]


def check_labels(X, C, g_labels, o_labels, best, second, rows=None):
    """Labels rule; returns the number of near-tie rows and of mismatches.

    ``rows`` maps the oracle's rows to rows of X (sampled parity); X and C are
    the full arrays. The band and the near-tie mask are the oracle's own
    (``oracle.tie_band``, ``oracle.near_ties``).
    """
    idx = np.arange(len(o_labels)) if rows is None else np.asarray(rows)
    g = g_labels[idx]
    assert g.min() >= 0 and g.max() < len(C)
    Xr = _rows_of(X, rows)
    band = oracle.tie_band(Xr, C, o_labels, TIE_RTOL)
    ties = oracle.near_ties(Xr, C, o_labels, best, second, TIE_RTOL)
    mism = np.nonzero(g != o_labels)[0]
    assert np.all(ties[mism]), (
        f"{len(mism)} label mismatches, {int((~ties[mism]).sum())} outside the near-tie band; "
        f"first rows {idx[mism[~ties[mism]]][:5]}")
    if len(mism):
        dg = exact_dist(X, C, idx[mism], g[mism])
        assert np.all(dg - best[mism] <= band[mism])
    return int(ties.sum()), int(len(mism))


def check_min_dist(X, C, g_labels, g_md, rows=None, o_labels=None, best=None):
    """min_dist rule. With the oracle's labels and best distances for these
    rows, rows where the GPU picked the oracle's label take ``best`` as the
    reference and only the others are recomputed."""
    idx = np.arange(len(X)) if rows is None else np.asarray(rows)
    g = g_labels[idx]
    if o_labels is not None:
        ref = np.array(best, dtype=np.float64, copy=True)
        diff_rows = np.nonzero(g != o_labels)[0]
        if len(diff_rows):
            ref[diff_rows] = exact_dist(X, C, idx[diff_rows], g[diff_rows])
    else:
        ref = exact_dist(X, C, idx, g)
    scale = sq_norms(_rows_of(X, rows)) + sq_norms(C)[g]
    err = np.abs(g_md[idx].astype(np.float64) - ref)
    ok = (err <= REL_TOL * ref) | (err <= TIE_RTOL * scale)
    assert np.all(ok), f"min_dist off on {int((~ok).sum())} rows, worst {err[~ok].max()}"
    assert np.all(g_md[idx] >= 0)


def exact_max_rows(n, k, d):
    """Clusters up to this size are summed by one wave in sample order on the
    GPU: 64 rows, or 128 when X has at least 2^26 elements and n >= 32 k."""
    return 128 if n * d >= 1 << 26 and n >= 32 * k else 64


def check_update(X, g_labels, C_old, g_Cnew, g_counts):
    """Update rules against the oracle's update on the GPU's labels. Returns
    the fraction of bit-exact centroid elements in the clusters summed in
    parts (above exact_max_rows)."""
    C_ref, cnt_ref, _ = oracle.update(X, g_labels, C_old)
    exact_rows = exact_max_rows(X.shape[0], C_old.shape[0], X.shape[1])
    assert np.array_equal(g_counts, cnt_ref), "counts differ"
    scale = np.abs(C_ref).max(axis=1, keepdims=True)
    err = np.abs(g_Cnew.astype(np.float64) - C_ref)
    assert np.all(err <= REL_TOL * scale), f"centroids off, worst {err.max()}"
    small = cnt_ref <= exact_rows
    assert np.array_equal(g_Cnew[small].view(np.uint32), C_ref[small].view(np.uint32)), \
        f"centroids of clusters with <= {exact_rows} rows not bit-exact against the in-order float64 mean"
    big = ~small
    if big.any():
        return float(np.mean(g_Cnew[big].view(np.uint32) == C_ref[big].view(np.uint32)))
    return 1.0


def check_counts_vs_oracle_labels(g_counts, o_labels, k, n_mismatch):
    o_counts = np.bincount(o_labels, minlength=k)
    diff = np.abs(g_counts - o_counts).sum()
    assert diff <= 2 * n_mismatch
    if n_mismatch == 0:
        assert np.array_equal(g_counts, o_counts)


def full_parity(X, C, min_dist=True):
    """The whole Lloyd step on the GPU against the oracle on every row."""
    g_labels, g_md, g_Cnew, g_counts = gpu_lloyd(X, C, min_dist=min_dist)
    o_labels, best, second = oracle.assign(X, C)
    ties, mism = check_labels(X, C, g_labels, o_labels, best, second)
    if min_dist:
        check_min_dist(X, C, g_labels, g_md)
    check_update(X, g_labels, C, g_Cnew, g_counts)
    check_counts_vs_oracle_labels(g_counts, o_labels, len(C), mism)
    return {"near_ties": ties, "mismatches": mism, "labels": g_labels}
