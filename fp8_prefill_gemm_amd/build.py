"""Ahead-of-time build of librz_fp8.so for gfx950 (hipcc, in-tree).

The library is the product: HIP kernels plus the C ABI declared in
include/rz_fp8.h.  It is compiled for gfx950 only, without fast-math, with
floating-point contraction off and IEEE fp32 division, and with packed fp32
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "librz_fp8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
SOURCES = ["api.hip", "kquant.hip", "actquant.hip", "gemm.hip", "gemm_edge.hip", "kgemv.hip", "kqgemm.hip",
           "q8gemm.hip"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile every HIP source into LIB_PATH (always rebuilds)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, "-I", os.path.join(ROOT, "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature name: drop that noise
    noise = ("unknown target feature", "packed-fp32-ops")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
