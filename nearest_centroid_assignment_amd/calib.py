"""Attainable-rate calibration on the GPU (context for the roofline).

``python -m nearest_centroid_assignment_amd.calib`` prints one JSON line with
* the fp32 MFMA rate of a kernel doing nothing but v_mfma_f32_32x32x2_f32 on
  four independent accumulators per wave, 8 waves per SIMD;
* the bandwidth of a streaming 16-byte copy of a 2 GiB buffer;
* the bandwidth of a streaming 16-byte read of a 4 GiB buffer (every byte
  read once; the ceiling of the update and k-means++ distance kernels, which
  mostly read), with ordinary and with non-temporal loads, at 512 to 2048
  blocks of 256 threads (the largest figure is reported as ``read_gbps``).
Both timed with HIP events on the launch stream (median of 5 after a warmup).
The published peaks (157.3 TFLOP/s fp32 matrix, 8 TB/s HBM) stay the roofline;
these numbers say how much of them the chip sustains here.
"""
from __future__ import annotations

import ctypes
import json
import os
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_PATH = os.path.join(HERE, "libkm_calib.so")
MFMA_FLOP = 2 * 32 * 32 * 2  # one v_mfma_f32_32x32x2_f32


def lib():
    if not os.path.exists(CALIB_PATH):
        raise RuntimeError(f"{CALIB_PATH} missing: run python -m nearest_centroid_assignment_amd.build")
    L = ctypes.CDLL(CALIB_PATH)
    L.km_calib_copy.restype = ctypes.c_int
    L.km_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.km_calib_read.restype = ctypes.c_int
    L.km_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_void_p]
    L.km_calib_mfma_f32.restype = ctypes.c_int
    L.km_calib_mfma_f32.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return L


def _time(fn, reps=5):
    import torch

    s = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    return statistics.median(out)


def copy_once(dst, src, nbytes, L=None):
    import torch

    L = L or lib()
    rc = L.km_calib_copy(dst.data_ptr(), src.data_ptr(), nbytes, torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"km_calib_copy returned {rc}")


def run(copy_bytes: int = 2 << 30, blocks: int = 256 * 8, iters: int = 20000,
        read_bytes: int = 4 << 30) -> dict:
    import torch

    L = lib()
    stream = torch.cuda.current_stream().cuda_stream
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")

    def mfma():
        if L.km_calib_mfma_f32(out.data_ptr(), blocks, iters, stream) != 0:
            raise RuntimeError("km_calib_mfma_f32 failed")

    t_mfma = _time(mfma)
    flop = blocks * 4 * iters * 4 * MFMA_FLOP
    src = torch.empty(copy_bytes, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    t_copy = _time(lambda: copy_once(dst, src, copy_bytes, L))
    del src, dst
    big = torch.ones(read_bytes // 4, dtype=torch.float32, device="cuda:0")
    reads = {}
    for nt in (0, 1):
        for rb in (256 * 2, 256 * 3, 256 * 4, 256 * 6, 256 * 8):
            sink = torch.empty(rb * 256, dtype=torch.float32, device="cuda:0")

            def read():
                if L.km_calib_read(big.data_ptr(), read_bytes, sink.data_ptr(), rb, nt,
                                   stream) != 0:
                    raise RuntimeError("km_calib_read failed")

            reads[f"{'nontemporal' if nt else 'ordinary'} {rb} blocks"] = \
                read_bytes / (_time(read) * 1e-3) / 1e9
    return {
        "read_gbps": max(reads.values()),
        "read_gbps_by_blocks": reads,
        "read_bytes": read_bytes,
        "mfma_f32_tflops": flop / (t_mfma * 1e-3) / 1e12,
        "mfma_ms": t_mfma,
        "copy_gbps": 2 * copy_bytes / (t_copy * 1e-3) / 1e9,
        "copy_ms": t_copy,
        "copy_bytes": copy_bytes,
    }


if __name__ == "__main__":
    print(json.dumps(run()), flush=True)
