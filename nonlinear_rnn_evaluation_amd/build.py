"""Builds libpnr.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree.

    python -m nonlinear_rnn_evaluation_amd.build          # or build_library() from Python

Every HIP translation unit is compiled with packed-FP32 code generation disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``); the kernels are written for
wave64 CDNA4 only.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpnr.so")
ARCH = os.environ.get("PNR_OFFLOAD_ARCH", "gfx950")

COMMON_FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found; libpnr needs the ROCm toolchain to build")


# host-code sanitizers for the checking build (device code is compiled as usual)
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
LIB_SANITIZED = os.path.join(HERE, "libpnr_san.so")


def build_library(verbose: bool = False, jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every HIP source and link libpnr.so; with sanitize, the host code is built
    with AddressSanitizer and UndefinedBehaviorSanitizer into libpnr_san.so instead (a
    checking build of the argument validation and workspace arithmetic, run on the CPU)."""
    hipcc = _hipcc()
    flags = COMMON_FLAGS + (SANITIZE_FLAGS if sanitize else [])
    lib = LIB_SANITIZED if sanitize else LIB
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = tempfile.mkdtemp(prefix="pnr_build_")
    try:
        def compile_one(src):
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [hipcc, *flags, "-c", src, "-o", obj]
            r = subprocess.run(cmd, capture_output=True, text=True)
            if r.returncode != 0:
                raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
            if verbose and r.stderr.strip():
                print(r.stderr, file=sys.stderr)
            return obj
        with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
            objs = list(ex.map(compile_one, srcs))
        out_tmp = lib + ".tmp"
        cmd = [hipcc, *flags, "-shared", *objs, "-o", out_tmp]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        os.replace(out_tmp, lib)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return lib


if __name__ == "__main__":
    print(build_library(verbose=True))
