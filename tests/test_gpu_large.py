"""GPU parity at sizes past 32-bit element counts: every index on these paths
must be 64-bit.  Inputs are generated on the device; the oracle checks
sampled rows, blocks and elements (first, last and random ones).

  - 1x128 and per-row quantization of X [524293, 4608] (2.4e9 elements);
  - 128x128 re-quantization of W [524416, 4608];
  - per-tensor quantization of a 2.4e9-element tensor whose maximum is planted
    (1000.0 at a known index, N(0, 1) elsewhere), so its scale is fixed by
    construction and sampled codes can be checked;
  - the block-scaled GEMM with an output of 131136 x 16384 > 2^31 elements;
  - a small-M GEMM with K past the 32-bit buffer offsets of its loads.
"""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_amd as fp8
import oracle
import synth
from tests.gpu_util import assert_rows_close, dev, ensure_library, host, sample_rows, say

pytestmark = pytest.mark.gpu

M_BIG, K_BIG = 524293, 4608  # M * K > 2^31


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


@pytest.fixture(scope="module")
def x_big():
    say(f"generating X [{M_BIG}, {K_BIG}] on the device")
    x = synth.normal_bf16((M_BIG, K_BIG), seed=71, device=dev())
    yield x
    del x
    torch.cuda.empty_cache()


def _rows(M):
    return sample_rows(M, 24, seed=M % 1000)


def test_block_quant_past_2e31_elements(x_big):
    say("quantize_block on 2.4e9 elements, sampled rows")
    q, s = fp8.quantize_block(x_big)
    rows = _rows(M_BIG)
    idx = torch.as_tensor(rows, device=dev())
    oq, os_ = oracle.quantize_block(x_big[idx].cpu())
    assert np.array_equal(host(q[idx]), oq)
    assert np.array_equal(host(s[idx]).view(np.uint32), os_.view(np.uint32))


def test_token_quant_past_2e31_elements(x_big):
    say("quantize_token on 2.4e9 elements, sampled rows")
    q, s = fp8.quantize_token(x_big)
    rows = _rows(M_BIG)
    idx = torch.as_tensor(rows, device=dev())
    oq, os_ = oracle.quantize_token(x_big[idx].cpu())
    assert np.array_equal(host(q[idx]), oq)
    assert np.array_equal(host(s[idx]).view(np.uint32), os_.view(np.uint32))


def test_tensor_quant_past_2e31_elements(x_big):
    say("quantize_tensor on 2.4e9 elements with a planted maximum")
    flat = x_big.view(-1)
    planted = flat.numel() - 77
    old = flat[planted].clone()
    flat[planted] = 1000.0
    try:
        q, s = fp8.quantize_tensor(x_big)
        picks = np.unique(np.concatenate([
            np.random.default_rng(5).integers(0, flat.numel(), 4000),
            [0, flat.numel() - 1, planted]]))
        pidx = torch.as_tensor(picks, device=dev())
        sample = flat[pidx].cpu()
        # the planted element is the maximum of the tensor (N(0, 1) elsewhere),
        # so the oracle's per-tensor quantization of the sample has its scale
        assert float(flat.float().abs().max().item()) == 1000.0
        oq, os_ = oracle.quantize_tensor(sample)
        assert host(s).view(np.uint32)[0] == np.asarray(os_).reshape(1).view(np.uint32)[0]
        assert np.array_equal(host(q.view(-1)[pidx]), oq)
    finally:
        flat[planted] = old


def test_requant_past_2e31_elements():
    N, K = 524416, K_BIG
    say(f"requantize_weights W [{N}, {K}], sampled block rows")
    w = synth.weight(N, K, seed=72, device=dev())
    (q, s), = fp8.requantize_weights([w], fp8.SCALE_F32)
    for br in (0, N // 128 - 1, 1717):
        wh = w[br * 128:(br + 1) * 128].cpu()
        oq, os_ = oracle.quantize_weight_block(wh, 0)
        assert np.array_equal(host(q[br * 128:(br + 1) * 128]), oq), f"block row {br}"
        assert np.array_equal(host(s[br:br + 1]).view(np.uint32), os_.view(np.uint32))
    del w, q, s
    torch.cuda.empty_cache()


def test_gemm_output_past_2e31_elements():
    M, N, K = 131136, 16384, 256
    say(f"block GEMM {M}x{N}x{K}: output past 2^31 elements, sampled rows")
    X = synth.act_col_outliers(M, K, seed=73, device=dev())
    W = synth.weight(N, K, seed=74, device=dev())
    qa, sa = fp8.quantize_block(X)
    (qw, sw), = fp8.requantize_weights([W], fp8.SCALE_F32)
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    rows = sample_rows(M, 12, seed=9)
    idx = torch.as_tensor(rows, device=dev())
    oqa, osa = oracle.quantize_block(X[idx].cpu())
    oqw, osw = oracle.quantize_weight_block(W.cpu(), 0)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_BLOCK)
    assert_rows_close(y, ref, rows=rows, what="large output")
    del X, W, qa, sa, qw, sw, y
    torch.cuda.empty_cache()


def test_small_m_gemm_k_past_buffer_offsets():
    """K = 2^22 + 128: 128 rows of K bytes no longer fit 32-bit buffer
    offsets, so the small-M kernels load with the global form."""
    M, N, K = 3, 128, (1 << 22) + 128
    say(f"block GEMM {M}x{N}x{K} (global-form loads)")
    X = synth.act_col_outliers(M, K, seed=75)
    W = synth.weight(N, K, seed=76, device=dev())
    qa, sa = fp8.quantize_block(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W], fp8.SCALE_F32)
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    oqa, osa = oracle.quantize_block(X)
    oqw, osw = oracle.quantize_weight_block(W.cpu(), 0)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_BLOCK)
    assert_rows_close(y, ref, what="long K")
    del W, qw, sw
    torch.cuda.empty_cache()
