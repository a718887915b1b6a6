"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/fp8w8a8.h declares, and its host-side validation returns the
documented status codes before touching the device (on a machine without a
GPU, valid arguments reach the device check and get FP8_ERR_DEVICE).
"""
import ctypes
import os
import re
import subprocess

import pytest

import fp8_w8a8_quantized_amd as fp8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8w8a8.h")

OK, ARG, SHAPE, ALIGN, DEVICE, LAUNCH = 0, -1, -2, -3, -4, -5


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fp8.library_path()):
        from fp8_w8a8_quantized_amd import build

        build.build()
    return fp8.load_library()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fp8_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_calls():
    names = _declared_functions()
    for required in ("fp8_quantize_block", "fp8_quantize_token", "fp8_rmsnorm_quant",
                     "fp8_requantize_weights", "fp8_gemm_a8w8_scaled",
                     "fp8_grouped_gemm_a8w8_scaled", "fp8_abi_version", "fp8_status_string",
                     "fp8_encode_f32_bits", "fp8_bf16_round_f32_bits",
                     "fp8_quantize_block_e8m0", "fp8_batched_gemm_a8w8_mxscale",
                     "fp8_quantize_tensors", "fp8_add_rmsnorm_quant", "fp8_swiglu_quant",
                     "fp8_silu_f32_of_bf16", "fp8_quantize_block_gather",
                     "fp8_inverse_rope_group_quant", "fp8_gemm_workspace_size",
                     "fp8_batched_gemm_mxscale_workspace_size", "fp8_build_source_hash",
                     "fp8_mfma_rate_probe"):
        assert required in names


def test_library_exports_every_declared_symbol(L):
    out = subprocess.run(["nm", "-D", "--defined-only", fp8.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(L, name)


def test_library_built_from_these_sources(L):
    from fp8_w8a8_quantized_amd import build

    assert L.fp8_build_source_hash().decode() == build.source_hash()


def test_version_and_status_strings(L):
    assert L.fp8_abi_version() == 3
    for st in (OK, ARG, SHAPE, ALIGN, DEVICE, LAUNCH):
        assert fp8.status_string(st) and fp8.status_string(st) != "unknown status"
    assert fp8.status_string(123) == "unknown status"


def _gpu():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


FAKE = 0x10000  # a 64 KiB-aligned non-null address, never dereferenced on error paths


def test_quantize_validation(L):
    vp = ctypes.c_void_p
    assert L.fp8_quantize_block(vp(FAKE), 4, 200, vp(FAKE), vp(FAKE), None) == SHAPE
    assert L.fp8_quantize_block(vp(FAKE), 4, 0, vp(FAKE), vp(FAKE), None) == SHAPE
    assert L.fp8_quantize_block(vp(FAKE), -1, 128, vp(FAKE), vp(FAKE), None) == ARG
    assert L.fp8_quantize_block(None, 4, 128, vp(FAKE), vp(FAKE), None) == ARG
    assert L.fp8_quantize_block(vp(FAKE + 2), 4, 128, vp(FAKE), vp(FAKE), None) == ALIGN
    assert L.fp8_quantize_block(vp(FAKE), 0, 128, None, None, None) == OK  # empty
    q8 = L.fp8_quantize_block_e8m0
    assert q8(vp(FAKE), 4, 200, vp(FAKE), vp(FAKE), None) == SHAPE
    assert q8(vp(FAKE), -1, 128, vp(FAKE), vp(FAKE), None) == ARG
    assert q8(vp(FAKE), 4, 128, vp(FAKE), None, None) == ARG
    assert q8(vp(FAKE), 4, 128, vp(FAKE + 4), vp(FAKE + 1), None) == ALIGN
    assert q8(vp(FAKE), 0, 128, None, None, None) == OK
    assert L.fp8_quantize_token(vp(FAKE), 4, 12, vp(FAKE), vp(FAKE), None) == SHAPE
    assert L.fp8_quantize_token(vp(FAKE), 4, 16, vp(FAKE), vp(FAKE + 1), None) == ALIGN
    assert L.fp8_rmsnorm_quant(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1e-6, 4, 16, 64,
                               None) == ARG
    assert L.fp8_rmsnorm_quant(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1e-6, 4, 136, 128,
                               None) == SHAPE
    assert L.fp8_rmsnorm_quant(vp(FAKE), vp(FAKE), vp(FAKE), None, 1e-6, 4, 16, 0, None) == ARG
    if not _gpu():
        assert L.fp8_quantize_block(vp(FAKE), 4, 128, vp(FAKE), vp(FAKE), None) == DEVICE
        assert q8(vp(FAKE), 4, 128, vp(FAKE), vp(FAKE + 1), None) == DEVICE
        assert L.fp8_rmsnorm_quant(vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE), 1e-6, 4, 16, 0,
                                   None) == DEVICE


def test_add_rmsnorm_quant_validation(L):
    vp = ctypes.c_void_p
    f, g = vp(FAKE), vp(FAKE + (1 << 20))
    add = L.fp8_add_rmsnorm_quant
    assert add(f, f, g, f, f, 1e-6, 4, 16, 64, None) == ARG          # group size
    assert add(f, f, g, f, f, 1e-6, 4, 136, 128, None) == SHAPE      # K % 128
    assert add(f, f, g, f, f, 1e-6, 4, 12, 0, None) == SHAPE         # K % 8
    assert add(f, f, None, f, f, 1e-6, 4, 16, 0, None) == ARG        # no residual
    assert add(f, f, vp(FAKE + (1 << 20) + 8), f, f, 1e-6, 4, 16, 0, None) == ALIGN
    assert add(f, f, vp(FAKE + 64), f, f, 1e-6, 4, 16, 0, None) == ARG  # x, residual overlap
    assert add(f, f, f, f, f, 1e-6, 4, 16, 0, None) == ARG              # same buffer
    assert add(f, f, g, f, f, 1e-6, 1 << 60, 16, 0, None) == SHAPE       # byte size overflows
    assert add(None, None, None, None, None, 1e-6, 0, 16, 0, None) == OK  # M == 0
    if not _gpu():
        assert add(f, f, g, f, f, 1e-6, 4, 16, 0, None) == DEVICE


def test_swiglu_validation(L):
    vp = ctypes.c_void_p
    f = vp(FAKE)
    assert L.fp8_swiglu_quant(f, -1, 128, f, f, None) == ARG
    assert L.fp8_swiglu_quant(f, 4, 100, f, f, None) == SHAPE
    assert L.fp8_swiglu_quant(f, 4, 0, f, f, None) == SHAPE
    assert L.fp8_swiglu_quant(f, 4, 128, None, f, None) == ARG
    assert L.fp8_swiglu_quant(vp(FAKE + 8), 4, 128, f, f, None) == ALIGN
    assert L.fp8_swiglu_quant(None, 0, 128, None, None, None) == OK
    assert L.fp8_silu_f32_of_bf16(0xFFFF, 2, f, None) == ARG
    assert L.fp8_silu_f32_of_bf16(0x10000, 0, f, None) == ARG
    assert L.fp8_silu_f32_of_bf16(0, 16, vp(FAKE + 2), None) == ALIGN
    if not _gpu():
        assert L.fp8_swiglu_quant(f, 4, 128, f, f, None) == DEVICE


def test_gather_validation(L):
    vp = ctypes.c_void_p
    f = vp(FAKE)
    g = L.fp8_quantize_block_gather
    assert g(f, 4, 128, f, -1, f, f, None) == ARG
    assert g(f, -1, 128, f, 4, f, f, None) == ARG
    assert g(f, 2 ** 31, 128, f, 4, f, f, None) == ARG
    assert g(f, 4, 100, f, 4, f, f, None) == SHAPE
    assert g(f, 4, 128, None, 4, f, f, None) == ARG
    assert g(None, 4, 128, f, 4, f, f, None) == ARG
    assert g(f, 4, 128, vp(FAKE + 2), 4, f, f, None) == ALIGN
    assert g(None, 0, 128, None, 0, None, None, None) == OK
    if not _gpu():
        assert g(f, 4, 128, f, 4, f, f, None) == DEVICE


def test_inverse_rope_validation(L):
    vp = ctypes.c_void_p
    f = vp(FAKE)
    r = L.fp8_inverse_rope_group_quant
    assert r(f, f, f, f, -1, 4, 128, 64, 16, 1, f, f, None) == ARG    # T
    assert r(f, f, f, f, 4, 4, 128, 63, 16, 1, f, f, None) == ARG     # odd rope dim
    assert r(f, f, f, f, 4, 4, 128, 64, 0, 1, f, f, None) == ARG      # no cache rows
    assert r(f, f, f, f, 4, 4, 128, 64, 16, 0, f, f, None) == ARG     # groups
    assert r(f, f, f, f, 4, 4, 100, 64, 16, 1, f, f, None) == SHAPE   # D % 8
    assert r(f, f, f, f, 4, 4, 64, 128, 16, 1, f, f, None) == SHAPE   # rope dim > D
    assert r(f, f, f, f, 4, 4, 128, 64, 16, 3, f, f, None) == SHAPE   # H % groups
    assert r(f, f, f, f, 4, 2, 96, 64, 16, 2, f, f, None) == SHAPE    # group width % 128
    assert r(f, None, f, f, 4, 4, 128, 64, 16, 1, f, f, None) == ARG
    assert r(f, f, None, f, 4, 4, 128, 64, 16, 1, f, f, None) == ARG
    assert r(f, vp(FAKE + 4), f, f, 4, 4, 128, 64, 16, 1, f, f, None) == ALIGN
    assert r(None, None, None, None, 0, 4, 128, 64, 16, 1, None, None, None) == OK
    if not _gpu():
        assert r(f, f, f, f, 4, 4, 128, 64, 16, 1, f, f, None) == DEVICE


def test_gemm_validation(L):
    vp = ctypes.c_void_p
    f = vp(FAKE)
    g = L.fp8_gemm_a8w8_scaled
    assert g(f, f, f, f, f, f, 16, 256, 256, 0, None, 0, None) == ARG  # bias
    assert g(f, f, f, f, None, f, 16, 200, 256, 0, None, 0, None) == SHAPE
    assert g(f, f, f, f, None, f, 16, 256, 200, 1, None, 0, None) == SHAPE
    assert g(f, f, f, f, None, f, 16, 256, 256, 7, None, 0, None) == ARG
    assert g(f, f, f, f, None, vp(FAKE + 8), 16, 256, 256, 0, None, 0, None) == ALIGN
    assert g(None, None, None, None, None, None, 0, 256, 256, 0, None, 0, None) == OK
    assert L.fp8_grouped_gemm_a8w8_scaled(f, f, f, f, f, f, 64, 0, 256, 256, None) == ARG
    assert L.fp8_grouped_gemm_a8w8_scaled(f, f, f, f, f, f, 64, 4, 256, 100, None) == SHAPE
    assert L.fp8_grouped_gemm_a8w8_scaled(f, f, f, f, f, f, 64, 1025, 256, 256, None) == ARG
    assert L.fp8_grouped_gemm_a8w8_scaled(f, f, f, f, f, f, 2**31, 4, 256, 256, None) == ARG
    assert L.fp8_grouped_gemm_a8w8_scaled(f, f, f, f, vp(FAKE + 2), f, 64, 4, 256, 256,
                                          None) == ALIGN
    mx = L.fp8_batched_gemm_a8w8_mxscale
    assert mx(f, f, f, f, f, 1, -1, 256, 256, None, 0, None) == ARG
    assert mx(f, f, f, f, f, -1, 16, 256, 256, None, 0, None) == ARG
    assert mx(f, f, f, f, f, 1, 16, 200, 256, None, 0, None) == SHAPE
    assert mx(f, f, f, f, f, 1, 16, 256, 200, None, 0, None) == SHAPE
    assert mx(f, f, f, f, f, 4, 16, 256, 1 << 21, None, 0, None) == SHAPE  # B * K > 2^22
    assert mx(f, f, f, f, vp(FAKE + 8), 1, 16, 256, 256, None, 0, None) == ALIGN
    assert mx(None, None, None, None, None, 1, 0, 256, 256, None, 0, None) == OK
    assert mx(None, None, None, None, None, 0, 16, 256, 256, None, 0, None) == OK
    if not _gpu():
        assert g(f, f, f, f, None, f, 16, 256, 256, 0, None, 0, None) == DEVICE
        assert mx(f, f, f, f, f, 1, 16, 256, 256, None, 0, None) == DEVICE


# Stream-K shapes: 128 x 128 tiles (M <= 128) or 256 x 128 tiles (M > 128 with
# >= 8 K steps per workgroup); the workspace is 256 workgroups x 2 partial
# slots of one tile's fp32 accumulators when a tile is split.
def test_gemm_workspace_sizes(L):
    ws = L.fp8_gemm_workspace_size
    slot1, slot2 = 128 * 128 * 4, 256 * 128 * 4
    assert ws(256, 6144, 4096, 0) == 256 * 2 * slot1   # qkv at decode: 128-row stream-K
    assert ws(256, 4096, 12288, 0) == 256 * 2 * slot2  # down: 256-row stream-K
    assert ws(256, 4096, 12288, 1) == 256 * 2 * slot2  # the row form takes the same plan
    assert ws(256, 24576, 4096, 0) == 0                # gate_up: 192 whole 256 x 128 tiles
    assert ws(100, 24576, 1024, 0) == 0                # 192 whole 128 x 128 tiles
    assert ws(129, 128, 128, 0) == 0                   # 2 tiles, 1 step each: no split
    assert ws(3, 1024, 12288, 0) == 256 * 2 * slot1    # 8 tiles x 96 steps over 256 ranks
    assert ws(8192, 24576, 4096, 0) == 0               # large-M kernel
    # N % 256 == 128 keeps even large M on the small-M kernels: 32 x 33 tiles of
    # 256 x 128 do not divide evenly over the CUs, so they are split
    assert ws(8192, 4224, 4096, 0) == 256 * 2 * slot2
    assert ws(0, 256, 256, 0) == 0
    assert ws(16, 200, 256, 0) == 0 and ws(16, 256, 256, 5) == 0  # refused arguments
    mxws = L.fp8_batched_gemm_mxscale_workspace_size
    assert mxws(1, 256, 4096, 12288) == 256 * 2 * slot2
    assert mxws(4, 256, 4096, 1024) == 0               # batched: the large-tile kernel
    assert mxws(1, 256, 4096, 200) == 0


def test_gemm_workspace_validation(L):
    vp = ctypes.c_void_p
    f = vp(FAKE)
    g = L.fp8_gemm_a8w8_scaled
    need = L.fp8_gemm_workspace_size(256, 4096, 12288, 0)
    assert need > 0
    assert g(f, f, f, f, None, f, 256, 4096, 12288, 0, None, 64, None) == ARG    # bytes, no ptr
    assert g(f, f, f, f, None, f, 256, 4096, 12288, 0, f, need - 16, None) == ARG  # too small
    assert g(f, f, f, f, None, f, 256, 4096, 12288, 0, vp(FAKE + 8), need, None) == ALIGN
    mx = L.fp8_batched_gemm_a8w8_mxscale
    assert mx(f, f, f, f, f, 1, 256, 4096, 12288, f, need - 1, None) == ARG
    if not _gpu():
        # a large enough workspace, or none at all, passes validation
        assert g(f, f, f, f, None, f, 256, 4096, 12288, 0, f, need, None) == DEVICE
        assert g(f, f, f, f, None, f, 256, 4096, 12288, 0, None, 0, None) == DEVICE
        assert mx(f, f, f, f, f, 1, 256, 4096, 12288, f, need, None) == DEVICE


def test_requant_validation(L):
    D = fp8._WeightDesc
    good = D(FAKE, FAKE, FAKE, 256, 256)
    bad_shape = D(FAKE, FAKE, FAKE, 200, 256)
    bad_align = D(FAKE + 4, FAKE, FAKE, 256, 256)
    arr = (D * 2)(good, bad_shape)
    assert L.fp8_requantize_weights(arr, 2, 0, None, 0, None) == SHAPE
    arr = (D * 2)(good, bad_align)
    assert L.fp8_requantize_weights(arr, 2, 1, None, 0, None) == ALIGN
    assert L.fp8_requantize_weights(arr, 2, 5, None, 0, None) == ARG
    assert L.fp8_requantize_weights(None, 0, 0, None, 0, None) == OK
    assert L.fp8_requantize_weights(None, -1, 0, None, 0, None) == ARG
    # workspace: none needed; a NULL one with a size, or a misaligned one, is refused
    for n in (-1, 0, 1, 64, 65, 10000):
        assert L.fp8_requantize_workspace_size(n) == 0
    arr = (D * 1)(good)
    assert L.fp8_requantize_weights(arr, 1, 0, None, 16, None) == ARG
    assert L.fp8_requantize_weights(arr, 1, 0, FAKE + 4, 16, None) == ALIGN
    if not _gpu():
        assert L.fp8_requantize_weights(arr, 1, 0, None, 0, None) == DEVICE
        assert L.fp8_requantize_weights(arr, 1, 0, FAKE, 256, None) == DEVICE


def test_tensor_quant_validation(L):
    vp = ctypes.c_void_p
    D = fp8._TensorDesc
    assert L.fp8_quantize_tensors(None, 0, None) == OK
    assert L.fp8_quantize_tensors(None, 1, None) == ARG
    assert L.fp8_quantize_tensors(None, -1, None) == ARG
    one = (D * 1)()
    one[0] = D(FAKE, FAKE, FAKE, 12)
    assert L.fp8_quantize_tensors(one, 1, None) == SHAPE
    one[0] = D(FAKE, FAKE, FAKE, -8)
    assert L.fp8_quantize_tensors(one, 1, None) == ARG
    one[0] = D(FAKE + 8, FAKE, FAKE, 64)
    assert L.fp8_quantize_tensors(one, 1, None) == ALIGN
    one[0] = D(FAKE, FAKE, FAKE + 2, 64)
    assert L.fp8_quantize_tensors(one, 1, None) == ALIGN
    one[0] = D(None, None, None, 0)
    assert L.fp8_quantize_tensors(one, 1, None) == OK  # empty tensor: skipped
    if not _gpu():
        one[0] = D(FAKE, FAKE, FAKE, 64)
        assert L.fp8_quantize_tensors(one, 1, None) == DEVICE


def test_encode_validation(L):
    vp = ctypes.c_void_p
    assert L.fp8_mfma_rate_probe(-1, vp(FAKE), None) == ARG
    assert L.fp8_mfma_rate_probe(4, None, None) == ARG
    assert L.fp8_mfma_rate_probe(4, vp(FAKE + 2), None) == ALIGN
    assert L.fp8_encode_f32_bits(1 << 32, 1, vp(FAKE), None) == ARG
    assert L.fp8_encode_f32_bits(0xFFFFFFFF, 2, vp(FAKE), None) == ARG
    assert L.fp8_encode_f32_bits(0, 16, vp(FAKE + 3), None) == ALIGN
    assert L.fp8_bf16_round_f32_bits(1 << 32, 1, vp(FAKE), None) == ARG
    assert L.fp8_bf16_round_f32_bits(0xFFFFFFFF, 2, vp(FAKE), None) == ARG
    assert L.fp8_bf16_round_f32_bits(0, 16, vp(FAKE + 2), None) == ALIGN
    assert L.fp8_bf16_round_f32_bits(0, 0, None, None) == OK


def test_quotient_path_equals_ieee_division_exhaustively(tmp_path):
    """The quantizers' reciprocal-corrected quotient equals IEEE x / s on every
    (bf16 x, bf16 amax) pair with |x| <= amax (host build of the same code)."""
    src = os.path.join(ROOT, "tests", "native", "quotient_check.cpp")
    exe = str(tmp_path / "quotient_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-mfma", src,
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "mismatches 0" in r.stdout


def test_fast_division_equals_integer_division(tmp_path):
    """The kernels' multiply-and-shift division of 31-bit group indices
    (fastdiv.hpp, host build of the same header) equals integer division."""
    src = os.path.join(ROOT, "tests", "native", "fastdiv_check.cpp")
    exe = str(tmp_path / "fastdiv_check")
    subprocess.run(["g++", "-O2", "-std=c++17", src, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 wrong" in r.stdout


# ---------------------------------------------- Python binding validation --
# Buffers passed by raw pointer are checked (dtype, exact shape, contiguity,
# device) before any call: a wrong buffer raises TypeError / ValueError on the
# host.  These run on CPU tensors; the device check comes last, so reaching it
# ("must be on a HIP device") means every other check passed.
import torch  # noqa: E402


def _cpu(shape, dtype):
    return torch.zeros(shape, dtype=dtype)


def test_binding_quantizer_out_checks():
    x = _cpu((4, 256), torch.bfloat16)
    good = (_cpu((4, 256), torch.uint8), _cpu((4, 2), torch.float32))
    with pytest.raises(ValueError, match="HIP device"):
        fp8.quantize_block(x, out=good)
    with pytest.raises(ValueError, match="shape"):
        fp8.quantize_block(x, out=(_cpu((4, 128), torch.uint8), good[1]))      # undersized q
    with pytest.raises(ValueError, match="shape"):
        fp8.quantize_block(x, out=(good[0], _cpu((4,), torch.float32)))        # row scales
    with pytest.raises(TypeError):
        fp8.quantize_block(x, out=(good[0], _cpu((4, 2), torch.float16)))      # dtype
    with pytest.raises(ValueError, match="contiguous"):
        fp8.quantize_block(x, out=(_cpu((256, 4), torch.uint8).t(), good[1]))
    with pytest.raises(ValueError, match="shape"):
        fp8.quantize_token(x, out=(good[0], _cpu((4, 2), torch.float32)))
    with pytest.raises(TypeError):
        fp8.quantize_block_e8m0(x, out=(good[0], _cpu((4, 2), torch.float32)))
    with pytest.raises(ValueError, match="shape"):
        fp8.rmsnorm_quant(x, _cpu((128,), torch.bfloat16))                    # gamma length
    with pytest.raises(ValueError, match="shape"):
        fp8.rmsnorm_quant(x, _cpu((256,), torch.bfloat16), group_size=128,
                          out=(good[0], _cpu((4,), torch.float32)))
    with pytest.raises(ValueError, match="shape"):
        fp8.add_rmsnorm_quant(x, _cpu((4, 128), torch.bfloat16), _cpu((256,), torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        fp8.swiglu_quant(x, out=(_cpu((4, 256), torch.uint8), _cpu((4, 1), torch.float32)))
    with pytest.raises(ValueError, match="shape"):
        fp8.quantize_block_gather(x, _cpu((3,), torch.int32),
                                  out=(_cpu((4, 256), torch.uint8), good[1]))
    with pytest.raises(ValueError, match="num_groups"):
        fp8.inverse_rope_group_quant(_cpu((2, 4, 128), torch.bfloat16), _cpu((2,), torch.int64),
                                     _cpu((16, 32), torch.float32), _cpu((16, 32), torch.float32),
                                     3)
    with pytest.raises(ValueError, match="shape"):
        fp8.inverse_rope_group_quant(_cpu((2, 4, 128), torch.bfloat16), _cpu((2,), torch.int64),
                                     _cpu((16, 32), torch.float32), _cpu((16, 16), torch.float32),
                                     1)
    with pytest.raises(ValueError, match="shape"):
        fp8.requantize_weights([_cpu((256, 256), torch.bfloat16)],
                               out=[(_cpu((256, 256), torch.uint8), _cpu((2, 1), torch.float32))])
    with pytest.raises(TypeError):
        fp8.requantize_weights([_cpu((256, 256), torch.bfloat16)], fp8.SCALE_E8M0,
                               out=[(_cpu((256, 256), torch.uint8), _cpu((2, 2), torch.float32))])
    with pytest.raises(ValueError, match="shape"):
        fp8.quantize_tensors([_cpu((4, 8), torch.bfloat16)],
                             out=[(_cpu((4, 8), torch.uint8), _cpu((2,), torch.float32))])


def test_binding_gemm_operand_checks():
    M, N, K = 16, 256, 512
    qa, qw = _cpu((M, K), torch.uint8), _cpu((N, K), torch.uint8)
    sa, sw = _cpu((M, K // 128), torch.float32), _cpu((N // 128, K // 128), torch.float32)
    with pytest.raises(ValueError, match="HIP device"):
        fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    with pytest.raises(ValueError, match="shape"):                       # row scales, block mode
        fp8.gemm_a8w8_scaled((qa, _cpu((M,), torch.float32)), (qw, sw), fp8.GRAN_BLOCK)
    with pytest.raises(ValueError, match="shape"):
        fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_ROW)
    with pytest.raises(ValueError, match="shape"):                       # w's K
        fp8.gemm_a8w8_scaled((qa, sa), (_cpu((N, K - 128), torch.uint8), sw), fp8.GRAN_BLOCK)
    with pytest.raises(TypeError):
        fp8.gemm_a8w8_scaled((qa, sa.double()), (qw, sw), fp8.GRAN_BLOCK)
    with pytest.raises(ValueError, match="shape"):                       # undersized out
        fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK,
                             out=_cpu((M, N - 128), torch.bfloat16))
    with pytest.raises(ValueError):
        fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), 5)
    with pytest.raises(ValueError, match="shape"):                       # grouped: w's K
        fp8.grouped_gemm_a8w8_scaled((qa, sa), (_cpu((2, N, 256), torch.uint8),
                                                 _cpu((2, 2, 2), torch.float32)),
                                     _cpu((3,), torch.int32))
    with pytest.raises(ValueError, match="shape"):                       # offsets length
        fp8.grouped_gemm_a8w8_scaled((qa, sa), (_cpu((2, N, K), torch.uint8),
                                                 _cpu((2, 2, 4), torch.float32)),
                                     _cpu((2,), torch.int32))
    with pytest.raises(ValueError, match="HIP device"):
        fp8.grouped_gemm_a8w8_scaled((qa, sa), (_cpu((2, N, K), torch.uint8),
                                                 _cpu((2, 2, 4), torch.float32)),
                                     _cpu((3,), torch.int32))
    sa8, sw8 = _cpu((M, K // 128), torch.uint8), _cpu((N // 128, K // 128), torch.uint8)
    with pytest.raises(ValueError, match="HIP device"):
        fp8.batched_gemm_a8w8_mxscale((qa, sa8), (qw, sw8))
    with pytest.raises(TypeError):                                       # fp32 scale bytes
        fp8.batched_gemm_a8w8_mxscale((qa, sa), (qw, sw8))
    with pytest.raises(ValueError, match="shape"):
        fp8.batched_gemm_a8w8_mxscale((qa.view(M, 1, K), sa8.view(M, 1, -1)),
                                      (_cpu((2, N, K), torch.uint8), _cpu((2, 2, 4), torch.uint8)))
