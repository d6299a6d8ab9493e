"""Build libgconv.so (gfx950) in-tree with hipcc.

    python -m depthwise_convolution_gconv_amd.build

Every HIP source is compiled for gfx950 only.  Packed-fp32 instructions are
disabled in device code (-Xclang -target-feature -Xclang -packed-fp32-ops); the
host pass warns that it does not know that feature, which is harmless.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libgconv.so")
# Measurement kernels of bench.py (MFMA-only loop, streaming copies): a library of
# their own, not part of the convolution boundary.
PEAKS_SRC = "peaks.hip"
PEAKS_LIB = os.path.join(PKG, "libgconv_peaks.so")

SOURCES = ["api.cpp", "direct2d.hip", "dw2d.hip", "dw1d_ntc.hip", "dw1d_wgrad.hip", "nhwc.hip", "igemm_nhwc.hip", "igemm.hip", "igemm_rows.hip", "igemm_defer.hip", "igemm_f32.hip"]
HEADERS = ["common.hpp", "fastdiv.hpp", "rows_common.hpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    path = os.path.join(CSRC, src)
    cmd = [HIPCC, f"--offload-arch={ARCH}", *FLAGS, "-c", path, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [HIPCC, *FLAGS, "-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libgconv.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    tmp = PEAKS_LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", *FLAGS, "-shared", os.path.join(CSRC, PEAKS_SRC), "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {PEAKS_SRC}:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, PEAKS_LIB)
    if verbose:
        print("built", LIB, "and", PEAKS_LIB)
    return LIB


def is_stale() -> bool:
    """True when libgconv.so is missing or older than a source or header."""
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, s) for s in SOURCES + HEADERS] + [os.path.join(INCLUDE, "gconv.h")]
    return any(os.path.getmtime(d) > t for d in deps)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
