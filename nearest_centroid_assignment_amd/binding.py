"""ctypes binding of ``libkmeans_mi355x.so`` (declared in include/kmeans_mi355x.h).

Argument marshalling only: torch tensors supply device pointers, the current
HIP stream and, when the caller passes none, the workspace allocation. Every
step of the computation runs in the library's HIP kernels. There is no CPU
fallback: if the library is missing, loading fails with an error.

The functions ``kmeans_assign``, ``kmeans_update``, ``kmeans_lloyd_step``,
``kmeans_lloyd_step_noalloc``, ``kmeans_fit``, ``kmeans_plusplus``, ``kmeans_workspace_bytes`` and
``kmeans_status_string`` mirror the C entry points of the same names;
``assign``, ``update``, ``lloyd_step``, ``fit`` and ``plusplus`` also allocate
the outputs.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkmeans_mi355x.so")

KM_OK = 0
KM_OP_ASSIGN, KM_OP_UPDATE, KM_OP_LLOYD, KM_OP_FIT, KM_OP_KMEANSPP = 0, 1, 2, 3, 4
KM_FIT_RELOCATE_EMPTY = 1
STATUS_NAMES = {
    0: "KM_OK",
    -1: "KM_ERR_NULL",
    -2: "KM_ERR_SHAPE",
    -3: "KM_ERR_ALIGN",
    -4: "KM_ERR_WORKSPACE",
    -5: "KM_ERR_ALIAS",
    -6: "KM_ERR_HIP",
    -7: "KM_ERR_OP",
    -8: "KM_ERR_SCRATCH",
}

_lock = threading.Lock()
_lib = None


class KMeansError(RuntimeError):
    """A C entry point returned a non-zero km_status."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: "
                         f"{kmeans_status_string(status)}")


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m nearest_centroid_assignment_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        i64, vp, sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
        L.kmeans_workspace_bytes.restype = sz
        L.kmeans_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int]
        L.kmeans_status_string.restype = ctypes.c_char_p
        L.kmeans_status_string.argtypes = [ctypes.c_int]
        L.kmeans_assign.restype = ctypes.c_int
        L.kmeans_assign.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
        L.kmeans_update.restype = ctypes.c_int
        L.kmeans_update.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
        L.kmeans_lloyd_step.restype = ctypes.c_int
        L.kmeans_lloyd_step.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp, sz, vp]
        L.kmeans_lloyd_step_noalloc.restype = ctypes.c_int
        L.kmeans_lloyd_step_noalloc.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, vp, vp]
        L.kmeans_plusplus.restype = ctypes.c_int
        L.kmeans_plusplus.argtypes = [vp, i64, i64, i64, i64, i64, vp, vp, vp, vp, sz, vp]
        L.kmeans_fit.restype = ctypes.c_int
        L.kmeans_fit.argtypes = [vp, vp, i64, i64, i64, i64, ctypes.c_double, ctypes.c_int,
                                 vp, vp, vp, vp, vp, vp, sz, vp]
        _lib = L
        return L


def kmeans_workspace_bytes(n: int, k: int, d: int, op: int) -> int:
    return int(lib().kmeans_workspace_bytes(n, k, d, op))


def kmeans_status_string(status: int) -> str:
    return lib().kmeans_status_string(status).decode()


# ----------------------------------------------------------- torch marshalling


def _torch():
    import torch

    return torch


def _ptr(t, dtype, shape, name):
    """Device pointer of a dense tensor of the given dtype and shape (None -> 0)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr() if t.numel() else None


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _side_stream(stream, device):
    """The torch stream the kernels go to when it is not the current stream
    (None otherwise, or when the caller passed a raw handle)."""
    torch = _torch()
    if isinstance(stream, torch.cuda.Stream) and stream != torch.cuda.current_stream(device):
        return stream
    return None


def _workspace(workspace, nbytes, device, stream=None):
    """The caller's workspace, or a new one. A new one is allocated on the
    stream the kernels run on, so the caching allocator does not hand its
    memory to other work before those kernels are done with it."""
    torch = _torch()
    if workspace is None:
        side = _side_stream(stream, device)
        if side is not None:
            with torch.cuda.stream(side):
                workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        else:
            workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    if workspace.dtype != torch.uint8 or workspace.device.type != "cuda":
        raise TypeError("workspace must be a uint8 GPU tensor")
    return workspace


def _record(stream, device, *tensors):
    """Mark tensors as used by a side stream: their memory is not reused until
    the work enqueued there so far is done (raw stream handles cannot be
    tracked; such callers keep the tensors alive themselves)."""
    side = _side_stream(stream, device)
    if side is not None:
        for t in tensors:
            if t is not None and t.numel():
                t.record_stream(side)


def _check(rc: int, where: str):
    if rc != KM_OK:
        raise KMeansError(rc, where)


def kmeans_assign(X, C, labels, min_dist=None, workspace=None, stream=None):
    """Enqueue the assignment of every row of X to its nearest row of C."""
    torch = _torch()
    n, d = X.shape
    k = C.shape[0]
    args = (_ptr(X, torch.float32, (n, d), "X"), _ptr(C, torch.float32, (k, d), "C"), n, k, d,
            _ptr(labels, torch.int64, (n,), "labels"),
            _ptr(min_dist, torch.float32, (n,), "min_dist"))
    workspace = _workspace(workspace, kmeans_workspace_bytes(n, k, d, KM_OP_ASSIGN), X.device,
                           stream)
    rc = lib().kmeans_assign(*args, workspace.data_ptr(), workspace.numel(),
                             _stream(stream, X.device))
    _check(rc, "kmeans_assign")
    _record(stream, X.device, X, C, labels, min_dist, workspace)


def kmeans_update(X, labels, C_old, C_new, counts, workspace=None, stream=None):
    """Enqueue the centroid update for fixed labels."""
    torch = _torch()
    n, d = X.shape
    k = C_old.shape[0]
    args = (_ptr(X, torch.float32, (n, d), "X"), _ptr(labels, torch.int64, (n,), "labels"),
            _ptr(C_old, torch.float32, (k, d), "C_old"), n, k, d,
            _ptr(C_new, torch.float32, (k, d), "C_new"), _ptr(counts, torch.int64, (k,), "counts"))
    workspace = _workspace(workspace, kmeans_workspace_bytes(n, k, d, KM_OP_UPDATE), X.device,
                           stream)
    rc = lib().kmeans_update(*args, workspace.data_ptr(), workspace.numel(),
                             _stream(stream, X.device))
    _check(rc, "kmeans_update")
    _record(stream, X.device, X, labels, C_old, C_new, counts, workspace)


def kmeans_lloyd_step(X, C_old, labels, min_dist, C_new, counts, workspace=None, stream=None):
    """Enqueue one Lloyd iteration (assignment against C_old, then update)."""
    torch = _torch()
    n, d = X.shape
    k = C_old.shape[0]
    args = (_ptr(X, torch.float32, (n, d), "X"), _ptr(C_old, torch.float32, (k, d), "C_old"),
            n, k, d, _ptr(labels, torch.int64, (n,), "labels"),
            _ptr(min_dist, torch.float32, (n,), "min_dist"),
            _ptr(C_new, torch.float32, (k, d), "C_new"), _ptr(counts, torch.int64, (k,), "counts"))
    workspace = _workspace(workspace, kmeans_workspace_bytes(n, k, d, KM_OP_LLOYD), X.device,
                           stream)
    rc = lib().kmeans_lloyd_step(*args, workspace.data_ptr(), workspace.numel(),
                                 _stream(stream, X.device))
    _check(rc, "kmeans_lloyd_step")
    _record(stream, X.device, X, C_old, labels, min_dist, C_new, counts, workspace)


def kmeans_lloyd_step_noalloc(X, C_old, labels, min_dist, C_new, counts, stream=None):
    """Enqueue one Lloyd iteration with the library's static scratch (no
    workspace; allocates nothing)."""
    torch = _torch()
    n, d = X.shape
    k = C_old.shape[0]
    args = (_ptr(X, torch.float32, (n, d), "X"), _ptr(C_old, torch.float32, (k, d), "C_old"),
            n, k, d, _ptr(labels, torch.int64, (n,), "labels"),
            _ptr(min_dist, torch.float32, (n,), "min_dist"),
            _ptr(C_new, torch.float32, (k, d), "C_new"), _ptr(counts, torch.int64, (k,), "counts"))
    rc = lib().kmeans_lloyd_step_noalloc(*args, _stream(stream, X.device))
    _check(rc, "kmeans_lloyd_step_noalloc")
    _record(stream, X.device, X, C_old, labels, min_dist, C_new, counts)


def kmeans_fit(X, C_init, max_iter, tol, flags, C_out, labels, min_dist, counts, info,
               workspace=None, stream=None):
    """Run Lloyd iterations (waits on the stream once per iteration)."""
    torch = _torch()
    n, d = X.shape
    k = C_init.shape[0]
    args = (_ptr(X, torch.float32, (n, d), "X"), _ptr(C_init, torch.float32, (k, d), "C_init"),
            n, k, d, int(max_iter), float(tol), int(flags),
            _ptr(C_out, torch.float32, (k, d), "C_out"), _ptr(labels, torch.int64, (n,), "labels"),
            _ptr(min_dist, torch.float32, (n,), "min_dist"),
            _ptr(counts, torch.int64, (k,), "counts"), _ptr(info, torch.float64, (3,), "info"))
    workspace = _workspace(workspace, kmeans_workspace_bytes(n, k, d, KM_OP_FIT), X.device,
                           stream)
    rc = lib().kmeans_fit(*args, workspace.data_ptr(), workspace.numel(),
                          _stream(stream, X.device))
    _check(rc, "kmeans_fit")
    _record(stream, X.device, X, C_init, C_out, labels, min_dist, counts, info, workspace)


def kmeans_plusplus(X, k, first, trials, rand, centres, chosen, workspace=None, stream=None):
    """Enqueue greedy k-means++ seeding with the given uniforms."""
    torch = _torch()
    n, d = X.shape
    args = (_ptr(X, torch.float32, (n, d), "X"), n, d, int(k), int(first), int(trials),
            _ptr(rand, torch.float64, (max(k - 1, 0) * trials,), "rand") if k > 1 else None,
            _ptr(centres, torch.float32, (k, d), "centres"), _ptr(chosen, torch.int64, (k,), "chosen"))
    workspace = _workspace(workspace, kmeans_workspace_bytes(n, k, d, KM_OP_KMEANSPP),
                           X.device, stream)
    rc = lib().kmeans_plusplus(*args, workspace.data_ptr(), workspace.numel(),
                               _stream(stream, X.device))
    _check(rc, "kmeans_plusplus")
    _record(stream, X.device, X, rand, centres, chosen, workspace)


# ------------------------------------------------------ allocating wrappers


def assign(X, C, min_dist: bool = True, stream=None):
    """Returns ``(labels, min_dist or None)`` as new GPU tensors."""
    torch = _torch()
    _ptr(X, torch.float32, X.shape, "X")
    n = X.shape[0]
    labels = torch.empty(n, dtype=torch.int64, device=X.device)
    md = torch.empty(n, dtype=torch.float32, device=X.device) if min_dist else None
    kmeans_assign(X, C, labels, md, stream=stream)
    return labels, md


def update(X, labels, C_old, stream=None):
    """Returns ``(C_new, counts)`` as new GPU tensors."""
    torch = _torch()
    C_new = torch.empty_like(C_old)
    counts = torch.empty(C_old.shape[0], dtype=torch.int64, device=X.device)
    kmeans_update(X, labels, C_old, C_new, counts, stream=stream)
    return C_new, counts


def lloyd_step(X, C_old, min_dist: bool = True, stream=None):
    """Returns ``(labels, min_dist or None, C_new, counts)`` as new GPU tensors."""
    torch = _torch()
    n, k = X.shape[0], C_old.shape[0]
    labels = torch.empty(n, dtype=torch.int64, device=X.device)
    md = torch.empty(n, dtype=torch.float32, device=X.device) if min_dist else None
    C_new = torch.empty_like(C_old)
    counts = torch.empty(k, dtype=torch.int64, device=X.device)
    kmeans_lloyd_step(X, C_old, labels, md, C_new, counts, stream=stream)
    return labels, md, C_new, counts


def fit(X, C_init, max_iter: int = 300, tol: float = 0.0, relocate_empty: bool = True,
        stream=None):
    """Lloyd iterations from C_init. Returns a dict of GPU tensors and numbers:
    centres, labels, min_dist, counts, n_iter, inertia, shift."""
    torch = _torch()
    n, k = X.shape[0], C_init.shape[0]
    C_out = torch.empty_like(C_init)
    labels = torch.empty(n, dtype=torch.int64, device=X.device)
    md = torch.empty(n, dtype=torch.float32, device=X.device)
    counts = torch.empty(k, dtype=torch.int64, device=X.device)
    info = torch.empty(3, dtype=torch.float64, device=X.device)
    kmeans_fit(X, C_init, max_iter, tol, KM_FIT_RELOCATE_EMPTY if relocate_empty else 0,
               C_out, labels, md, counts, info, stream=stream)
    # info is read on the host: wait for the stream the fit ran on.
    if stream is None or isinstance(stream, torch.cuda.Stream):
        (stream or torch.cuda.current_stream(X.device)).synchronize()
    else:
        torch.cuda.synchronize(X.device)
    n_iter, inertia, shift = info.cpu().tolist()
    return {"centres": C_out, "labels": labels, "min_dist": md, "counts": counts,
            "n_iter": int(n_iter), "inertia": inertia, "shift": shift}


def plusplus(X, k, first, trials, rand, stream=None):
    """Returns (centres, chosen) of greedy k-means++ seeding as GPU tensors;
    rand is a (k - 1, trials) or flat float64 GPU tensor of uniforms."""
    torch = _torch()
    d = X.shape[1]
    centres = torch.empty((k, d), dtype=torch.float32, device=X.device)
    chosen = torch.empty(k, dtype=torch.int64, device=X.device)
    r = rand.reshape(-1) if rand is not None and k > 1 else None
    kmeans_plusplus(X, k, first, trials, r, centres, chosen, stream=stream)
    return centres, chosen
