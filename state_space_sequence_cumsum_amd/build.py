"""Compile libssd.so (HIP kernels + C ABI) for gfx950, in-tree, with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBRARY = os.path.join(PKG, "libssd.so")
SOURCES = [os.path.join(CSRC, "ssd_kernels.hip"), os.path.join(CSRC, "ssd_bf16.hip"),
           os.path.join(CSRC, "ssd_step.hip"), os.path.join(CSRC, "ssd_noalloc.hip"),
           os.path.join(CSRC, "ssd_small.hip"),
           os.path.join(CSRC, "ssd_api.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler from forming packed fp32 VALU ops (v_pk_fma_f32 and friends)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: scaling a running state in place then
    # needs no accumulator-register round trips
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def hipcc() -> str:
    cand = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cand):
        raise RuntimeError("hipcc not found; the ROCm toolchain is required to build libssd")
    return cand


def build(verbose: bool = False) -> str:
    tmp = LIBRARY + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
