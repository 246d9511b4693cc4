"""Build ``libkmeans_mi355x.so`` (the C-ABI HIP library) in-tree for gfx950.

Usage: ``python -m nearest_centroid_assignment_amd.build [--save-temps]``.
hipcc cross-compiles without a GPU, so this runs on any host with ROCm.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libkmeans_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "assign.hip", "update.hip", "fit.hip", "kmeanspp.hip"]
# Calibration kernels for the measurements (copy, MFMA loop): a separate library.
CALIB_NAME = "libkm_calib.so"
CALIB_PATH = os.path.join(HERE, CALIB_NAME)
CALIB_SOURCES = ["calib.hip"]

# Per-source additional flags. The assignment kernel uses LLVM's iterative
# occupancy-driven scheduler (measured, same-box A/B on the large shapes:
# 0.8-0.9 % faster than the max-ilp strategy, which was itself 1-2 % faster
# than the default; max-memory-clause, iterative-ilp and iterative-minreg
# were 0.3-3 % slower).
EXTRA_FLAGS: dict[str, list[str]] = {
    "assign.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-maxocc"],
}

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # No packed-FP32 instructions in generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _run(cmd, cwd=None, verbose=False):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    # The host pass warns that it does not know the packed-fp32 feature; that
    # warning is expected. Anything else is shown.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    msgs = [l for l in (proc.stdout + proc.stderr).splitlines() if noise not in l and l.strip()]
    if msgs and (verbose or proc.returncode):
        print("\n".join(msgs), file=sys.stderr)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed with exit code {proc.returncode}: {' '.join(cmd)}")


def _compile(sources, out_path, verbose: bool, save_temps: bool, extra_flags=None) -> str:
    """Compile each source to an object (in parallel), then link the library.

    ``extra_flags`` maps a source name to additional hipcc flags for it.
    """
    from concurrent.futures import ThreadPoolExecutor

    extra_flags = extra_flags or {}
    objdir = os.path.join(HERE, "..", "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]

    def one(src):
        obj = os.path.join(objdir, os.path.basename(out_path) + "." + src + ".o")
        cmd = [hipcc(), *compile_flags, *extra_flags.get(src, []), "-c", "-o", obj,
               os.path.join(CSRC, src)]
        if save_temps:
            cmd.insert(1, "-save-temps")
        _run(cmd, cwd=objdir, verbose=verbose)
        return obj

    with ThreadPoolExecutor(max_workers=len(sources)) as pool:
        objs = list(pool.map(one, sources))
    out_tmp = out_path + ".tmp"
    _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out_tmp, *objs],
         verbose=verbose)
    os.replace(out_tmp, out_path)
    return out_path


def build(verbose: bool = False, save_temps: bool = False) -> str:
    """Compile the k-means library and the calibration library; returns the
    path of the k-means library."""
    _compile(CALIB_SOURCES, CALIB_PATH, verbose, save_temps)
    return _compile(SOURCES, LIB_PATH, verbose, save_temps, EXTRA_FLAGS)


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
