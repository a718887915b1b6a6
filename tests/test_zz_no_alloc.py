"""The allocation-free GEMM entry point (fp8_gemm_a8w8_scaled_noalloc),
through the C ABI: its output equals fp8_gemm_a8w8_scaled's (given a workspace
of the queried size) byte for byte, and both are within the GEMM tolerance of
the oracle.  Two calls in a row share the library's scratch array; the second
is smaller and splits fewer, smaller partial tiles, so stale partials of the
first call would show up in it."""
import ctypes

import pytest
import torch

import fp8_w8a8_quantized_amd as fp8
import oracle
import synth
from tests.gpu_util import assert_gemm_all_rows, dev, ensure_library, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _vp(t):
    return ctypes.c_void_p(t.data_ptr())


def _operands(M, N, K, seed, gran):
    X = synth.act_col_outliers(M, K, seed=seed)
    W = synth.weight(N, K, seed=seed + 1)
    if gran == fp8.GRAN_BLOCK:
        qa, sa = fp8.quantize_block(X.to(dev()))
        (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
        oqa, osa = oracle.quantize_block(X)
        oqw, osw = oracle.quantize_weight_block(W, 0)
    else:
        qa, sa = fp8.quantize_token(X.to(dev()))
        qw, sw = fp8.quantize_token(W.to(dev()))
        oqa, osa = oracle.quantize_token(X)
        oqw, osw = oracle.quantize_token(W)
    return (qa, sa, qw, sw), (oqa, osa, oqw, osw)


def _with_workspace(L, ops, M, N, K, gran, st):
    qa, sa, qw, sw = ops
    need = L.fp8_gemm_workspace_size(M, N, K, gran)
    ws = torch.empty((max(need, 16),), dtype=torch.uint8, device=dev())
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    rc = L.fp8_gemm_a8w8_scaled(_vp(qa), _vp(qw), _vp(sa), _vp(sw), None, _vp(y), M, N, K, gran,
                                _vp(ws), ws.numel(), st)
    assert rc == 0
    torch.cuda.synchronize()
    return y


def _noalloc(L, ops, M, N, K, gran, st):
    qa, sa, qw, sw = ops
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    rc = L.fp8_gemm_a8w8_scaled_noalloc(_vp(qa), _vp(qw), _vp(sa), _vp(sw), None, _vp(y), M, N,
                                        K, gran, st)
    assert rc == 0
    torch.cuda.synchronize()
    return y


# first: 256-row stream-K with split tiles (the full 64 MiB of partials);
# second, smaller: 128-row stream-K over 8 tiles of 96 K steps, row scales
CASES = [((256, 4096, 12288), fp8.GRAN_BLOCK), ((3, 1024, 12288), fp8.GRAN_ROW)]


def test_noalloc_gemm_matches_workspace_entry_point_twice():
    L = fp8.load_library()
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for (M, N, K), gran in CASES:
        assert L.fp8_gemm_workspace_size(M, N, K, gran) > 0  # a split plan: scratch is used
    for i, ((M, N, K), gran) in enumerate(CASES):
        say(f"no-alloc GEMM call {i}: {M}x{N}x{K} gran {gran}")
        ops, ref_ops = _operands(M, N, K, seed=500 + 10 * i, gran=gran)
        y_ref = _with_workspace(L, ops, M, N, K, gran, st)
        y = _noalloc(L, ops, M, N, K, gran, st)
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"call {i}"
        assert_gemm_all_rows(y, *ref_ops, gran, what=f"no-alloc call {i}")


def test_noalloc_gemm_validation():
    L = fp8.load_library()
    f = ctypes.c_void_p(0x10000)
    g = L.fp8_gemm_a8w8_scaled_noalloc
    assert g(f, f, f, f, f, f, 16, 256, 256, 0, None) == -1            # bias
    assert g(f, f, f, f, None, f, 16, 200, 256, 0, None) == -2         # N % 128
    assert g(f, f, f, f, None, ctypes.c_void_p(0x10008), 16, 256, 256, 0, None) == -3
    assert g(None, None, None, None, None, None, 0, 256, 256, 0, None) == 0
