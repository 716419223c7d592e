"""Build libxt.so (HIP kernels + C ABI + tape) for gfx950 with hipcc.

    python autograd_row_wise_amd/build.py      # writes autograd_row_wise_amd/libxt.so

Every source is compiled every time (in parallel), then linked.  The packed
FP32 target feature is turned off for all device code (hipcc's host pass
warns that it does not know the feature; that is expected).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libxt.so")
SOURCES = ["abi.cpp", "tape.cpp", "rowwise.hip", "rowstream.hip", "ce.hip", "elementwise.hip", "rope.hip", "gemm.hip", "gradbuf.hip", "embed.hip", "attention.hip", "noalloc.hip"]
ARCH = os.environ.get("XT_OFFLOAD_ARCH", "gfx950")

FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]
# Per-source additions.  attention.hip: matrix-core accumulators in ordinary
# VGPRs, so the softmax of a score tile reads them without AGPR copies.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found; libxt needs ROCm to build")
    return h


def _compile(src: str, obj: str) -> None:
    cmd = [_hipcc(), *FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), [])]
    if src.endswith(".cpp"):
        cmd += ["-x", "hip"]
    cmd += ["-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{r.stderr}")


def build(verbose: bool = True) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for s in SOURCES:
        jobs.append((os.path.join(CSRC, s), os.path.join(objdir, s + ".o")))
    workers = min(len(jobs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(lambda j: _compile(*j), jobs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for _, o in jobs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking libxt.so failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
