"""Build libqmm.so in-tree with hipcc for gfx950.

    python -m quantized_matmul_ggml_amd.build

Flags: -O3, no fast-math (the quantizer needs IEEE division and
round-to-nearest-even conversions to be bit-exact), and packed fp32
instructions disabled in device code.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqmm.so")
SOURCES = ["qmm_api.cpp", "quant.hip", "gemv.hip", "gemv_i8.hip", "gemv_mf.hip",
           "gemm.hip", "gemm_rq.hip", "records.hip", "probe.hip"]
ARCH = os.environ.get("QMM_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fvisibility=hidden", "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-Wno-unused-command-line-argument"]


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every source into one shared library (always recompiles)."""
    srcs = []
    for s in SOURCES:
        srcs += ["-x", "hip", os.path.join(CSRC, s)]
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
