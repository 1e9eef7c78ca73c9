"""Builds libtq2.so in-tree with hipcc for gfx950.

Flags: -O3, C++17, position-independent shared object; packed-FP32 VALU ops are
disabled for the device code (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libtq2.so")
SOURCES = ["libtq2.cpp", "repack.cpp", "tq2_gemv.hip", "mfma_gemm.hip", "blr.hip", "skinny_gemm.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def compile_cmd(out: str, extra=()) -> list:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-x", "hip", *srcs,
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-result", *extra, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = compile_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
