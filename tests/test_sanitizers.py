"""Host sanitizer builds (no GPU): the CPU oracle and the C ABI's host-side
validation, compiled with AddressSanitizer and UndefinedBehaviorSanitizer
(every report fatal), each driven by a native program that calls every
function on edge inputs held in exactly sized buffers.

  * oracle: gcc build of oracle/fp8_oracle.c + tests/native/oracle_sanitize.c
    (every oracle function; results the number formats fix on their own);
  * ABI: hipcc build of the library's sources + tests/native/abi_sanitize.cpp
    with the sanitizers on the host side only (device code is not
    instrumented), calling every entry point with arguments that must be
    refused, sizes whose byte counts would overflow, and valid ones that
    stop at the device check on a machine without a GPU.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "fp8_w8a8_quantized_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _run(exe, env_extra):
    env = dict(os.environ, **env_extra)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-ffp-contract=off",
                    "-fopenmp", os.path.join(ROOT, "oracle", "fp8_oracle.c"),
                    os.path.join(NATIVE, "oracle_sanitize.c"), "-o", exe, "-lm"], check=True)
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=1"})


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_abi_validation_under_asan_ubsan(tmp_path):
    from fp8_w8a8_quantized_amd import build

    if not os.path.exists(build.SILU_INC):  # generated at build time
        build.gen_silu_table()
    exe = str(tmp_path / "abi_sanitize")
    srcs = [os.path.join(CSRC, f) for f in ("api.hip", "quant.hip", "gemm.hip")]
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", *srcs, os.path.join(NATIVE, "abi_sanitize.cpp"),
                    "-o", exe], check=True, capture_output=True)
    # the HIP runtime is not instrumented and keeps process-lifetime state
    _run(exe, {"ASAN_OPTIONS": "detect_leaks=0"})
