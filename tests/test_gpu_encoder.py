"""The device E4M3 encoder (used by every quantizer) and the device bf16
rounding (RMSNorm output, every bf16 GEMM output) against the oracle on all
2^32 fp32 bit patterns.  NaN inputs are outside the contract and are not
compared; infinities saturate (E4M3) or stay infinite (bf16) on both sides."""
import numpy as np
import pytest

import fp8_w8a8_quantized_amd as fp8
import oracle
from tests.gpu_util import ensure_library, host, say

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_encoder_all_fp32_patterns():
    ensure_library()
    step = 1 << 28
    for lo in range(0, 1 << 32, step):
        say(f"encode fp32 patterns [{lo:#x}, {lo + step:#x})")
        g = host(fp8.encode_f32_bits(lo, step))
        bits = np.arange(lo, lo + step, dtype=np.uint64).astype(np.uint32)
        ref = oracle.e4m3_encode_array(bits.view(np.float32))
        nan = ((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x7FFFFF) != 0)
        bad = np.nonzero((g != ref) & ~nan)[0]
        assert bad.size == 0, (f"{bad.size} mismatches, first patterns "
                               f"{[hex(int(bits[i])) for i in bad[:6]]} gpu "
                               f"{[hex(int(g[i])) for i in bad[:6]]} oracle "
                               f"{[hex(int(ref[i])) for i in bad[:6]]}")


@pytest.mark.timeout(900)
def test_bf16_rounding_all_fp32_patterns():
    ensure_library()
    step = 1 << 28
    for lo in range(0, 1 << 32, step):
        say(f"bf16-round fp32 patterns [{lo:#x}, {lo + step:#x})")
        g = host(fp8.bf16_round_f32_bits(lo, step)).view(np.uint16)
        bits = np.arange(lo, lo + step, dtype=np.uint64).astype(np.uint32)
        ref = oracle.bf16_rne_array(bits.view(np.float32))
        nan = ((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x7FFFFF) != 0)
        bad = np.nonzero((g != ref) & ~nan)[0]
        assert bad.size == 0, (f"{bad.size} mismatches, first patterns "
                               f"{[hex(int(bits[i])) for i in bad[:6]]} gpu "
                               f"{[hex(int(g[i])) for i in bad[:6]]} oracle "
                               f"{[hex(int(ref[i])) for i in bad[:6]]}")
