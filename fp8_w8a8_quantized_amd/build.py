"""Build libfp8w8a8.so (HIP, gfx950) in-tree with hipcc.

Flags:
  --offload-arch=gfx950                 MI355X only
  -ffp-contract=off                     no implicit FMA: every fp32 operation the
                                        quantizers' definitions name is one
                                        rounding (explicit fmaf is still an FMA)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                        no packed fp32 instructions
fp32 denormals stay enabled (hipcc's default; no flush flag is passed), and
divisions and square roots stay correctly rounded (hipcc's default).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8w8a8.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``fp8_w8a8_quantized_amd/libfp8w8a8.so``."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
