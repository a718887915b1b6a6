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

import hashlib
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8w8a8.so")
SOURCES = ["api.hip", "quant.hip", "gemm.hip"]
INCLUDE = os.path.join(os.path.dirname(HERE), "include", "fp8w8a8.h")
HASH_TAG = b"FP8W8A8_SOURCE_SHA256="

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def source_hash() -> str:
    """SHA-256 over every file the library is built from (csrc/ and the C
    header), in name order."""
    h = hashlib.sha256()
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                   if f.endswith((".hip", ".hpp", ".h", ".c")))
    for path in files + [INCLUDE]:
        h.update(os.path.basename(path).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def built_hash(lib: str = LIB):
    """The source hash recorded in a built library (None if absent)."""
    try:
        with open(lib, "rb") as f:
            m = re.search(re.escape(HASH_TAG) + rb"([0-9a-f]{64})", f.read())
    except OSError:
        return None
    return m.group(1).decode() if m else None


def is_current(lib: str = LIB) -> bool:
    """True when ``lib`` exists and was built from the sources as they are."""
    return built_hash(lib) == source_hash()


SILU_GEN = os.path.join(CSRC, "gen_silu_table.c")
SILU_INC = os.path.join(CSRC, "silu_table.inc")


def gen_silu_table(verbose: bool = False) -> str:
    """Build step: compile and run gen_silu_table.c (gcc, libquadmath), which
    writes csrc/silu_table.inc, the SwiGLU kernel's table of correctly rounded
    silu values over the middle band of bf16 inputs (it also checks the
    kernel's closed forms on every other finite input)."""
    exe = os.path.join(CSRC, "_gen_silu_table")
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", SILU_GEN, "-o", exe, "-lquadmath", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    try:
        subprocess.run([exe, SILU_INC + ".tmp"], check=True)
        os.replace(SILU_INC + ".tmp", SILU_INC)
    finally:
        os.remove(exe)
    return SILU_INC


def build(verbose: bool = False) -> str:
    """Compile every HIP source into ``fp8_w8a8_quantized_amd/libfp8w8a8.so``,
    recording the sources' hash in it (fp8_build_source_hash)."""
    gen_silu_table(verbose)
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, f'-DFP8W8A8_SOURCE_SHA256="{source_hash()}"', *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
