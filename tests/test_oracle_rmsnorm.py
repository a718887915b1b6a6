"""Pins for the oracle's RMSNorm and fused RMSNorm + per-token quantization.

The fixed fp32 summation order is a definition (the pages fix none), so the
order itself is pinned only by self-consistency; everything around it is
pinned by: closed forms (x == 1, equal magnitudes), the exact sum of squares
within the fp32 error bound of the fixed order, agreement with
torch.nn.functional.rms_norm in fp64 (the definition the page cites) to one
bf16 ulp, the bf16 rounding against torch's dtype conversion, and the fused ==
composed identity.  The residual add of the fused add + RMSNorm is pinned by
exact rational arithmetic (crafted ties, wide exponent gaps, subnormals), by
torch's bf16 add, and by its identities (r == 0, r == -x).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from _exact import frac_to_bf16_bits


def _f32(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def test_bf16_rounding_matches_torch_conversion():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))).astype(np.float32)
    # exact ties: bf16 value + half an ulp
    base = (rng.integers(0x3000, 0x4F00, 2000).astype(np.uint32) << 16)
    ties = (base | 0x8000).view(np.float32)
    allv = np.concatenate([v, ties, -ties])
    ref = torch.from_numpy(allv).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16_rne(float(x)) for x in allv], np.uint16)
    assert np.array_equal(got, ref)


def test_ones_closed_form():
    K = 5120
    x = np.full((3, K), 0x3F80, np.uint16)  # 1.0
    g = np.full(K, 0x3F80, np.uint16)
    assert oracle.rms_sumsq(x[0]) == float(K)
    y = oracle.rmsnorm_bf16(x, g, 1e-6)
    assert np.all(y == 0x3F80)  # 1/sqrt(1 + 1e-6) rounds to 1.0 in bf16
    q, s = oracle.rmsnorm_quant(x, g, 1e-6)
    assert np.all(q == 0x7E)
    assert np.all(s == np.float32(1.0) / np.float32(448.0))


def test_equal_magnitudes_quantize_to_max():
    K = 1024
    rng = np.random.default_rng(3)
    sign = np.where(rng.random((4, K)) < 0.5, 0x8000, 0).astype(np.uint16)
    x = (sign | np.uint16(0x4040)).astype(np.uint16)  # +-3.0
    g = np.full(K, 0x3F80, np.uint16)
    q, s = oracle.rmsnorm_quant(x, g, 1e-6)
    assert np.array_equal(q, np.where(sign != 0, 0xFE, 0x7E).astype(np.uint8))


@pytest.mark.parametrize("K", [8, 64, 520, 5120])
def test_fixed_order_sum_within_fp32_bound_of_exact(K):
    rng = np.random.default_rng(K)
    for trial in range(5):
        x = synth.bf16_bits(synth.to_bf16(rng.standard_normal(K).astype(np.float32) *
                                          np.exp2(rng.integers(-8, 8, K)).astype(np.float32)))
        xf = _f32(x)
        exact = sum(Fraction(float(v)) ** 2 for v in xf)
        got = Fraction(oracle.rms_sumsq(x))
        # each fp32 addition adds at most one rounding of relative 2^-24
        assert abs(got - exact) <= (K - 1) * Fraction(1, 2 ** 24) * exact * Fraction(11, 10)


def test_bf16_rne_array_matches_torch_conversion():
    """The array form (used against the device rounding on all 2^32 patterns)
    equals torch's fp32 -> bf16 conversion (round to nearest even) on every
    1021st fp32 pattern, on exact ties and on subnormals; NaNs excluded."""
    bits = np.arange(0, 1 << 32, 1021, dtype=np.uint64).astype(np.uint32)
    ties = (np.arange(0, 1 << 16, dtype=np.uint32) << 16) | 0x8000
    sub = np.arange(1, 1 << 23, 4099, dtype=np.uint32)
    bits = np.concatenate([bits, ties, ties | 0x80000000, sub, sub | 0x80000000])
    bits = bits[~(((bits & 0x7F800000) == 0x7F800000) & ((bits & 0x7FFFFF) != 0))]
    v = bits.view(np.float32)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne_array(v)
    assert np.array_equal(got, ref)


def test_matches_torch_rms_norm_in_fp64_within_one_bf16_ulp():
    h, gamma = synth.rms_inputs(M=64, K=5120, seed=2)
    y = oracle.rmsnorm_bf16(h, gamma, 1e-6)
    ref = torch.nn.functional.rms_norm(h.double(), (5120,), weight=gamma.double(), eps=1e-6)
    ref_b = ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).astype(np.int32)
    yi = y.astype(np.int32)
    # same sign, bf16 patterns differ by at most one step
    assert np.all(np.abs(yi - ref_b) <= 1)
    assert np.mean(yi == ref_b) > 0.99


def test_fused_equals_composed():
    h, gamma = synth.rms_inputs(M=32, K=5120, seed=4)
    qf, sf = oracle.rmsnorm_quant(h, gamma, 1e-6)
    y = oracle.rmsnorm_bf16(h, gamma, 1e-6)
    qc, sc = oracle.quantize_token(y)
    assert np.array_equal(qf, qc) and np.array_equal(sf, sc)


def _bf16_pairs(n, seed):
    """Random finite bf16 pairs with exponent gaps 0..60, mixed signs, plus
    crafted exact ties, cancellations and subnormals (uint16 bits)."""
    rng = np.random.default_rng(seed)
    ex = rng.integers(0x30, 0x90, n).astype(np.uint32)
    gap = rng.integers(0, 61, n).astype(np.uint32)
    ey = np.clip(ex.astype(np.int64) - gap, 1, 254).astype(np.uint32)
    sx = rng.integers(0, 2, n).astype(np.uint32) << 15
    sy = rng.integers(0, 2, n).astype(np.uint32) << 15
    x = sx | (ex << 7) | rng.integers(0, 128, n).astype(np.uint32)
    y = sy | (ey << 7) | rng.integers(0, 128, n).astype(np.uint32)
    # ties: 1 + m/128 plus 2^-8 (half an ulp) -> even neighbour
    m = np.arange(128, dtype=np.uint32)
    tx = (127 << 7) | m
    ty = np.full(128, 0x3B80, np.uint32)  # 2^-8
    # cancellation to exact zero and to a few ulps
    cx = x[:64]
    cy = cx ^ 0x8000
    dx = x[64:128]
    dy = (dx ^ 0x8000) + 1
    # subnormal bf16 operands and sums
    sub = rng.integers(1, 128, 64).astype(np.uint32)
    sub2 = rng.integers(1, 128, 64).astype(np.uint32) | 0x8000 * rng.integers(0, 2, 64).astype(
        np.uint32)
    xs = np.concatenate([x, tx, cx, dx, sub, (1 << 7) | sub]).astype(np.uint16)
    ys = np.concatenate([y, ty, cy, dy, sub2, sub2]).astype(np.uint16)
    return xs, ys


def test_add_bf16_against_exact_rationals():
    """Every sum is the nearest bf16 to the exact rational x + r, found by
    exact comparison (ties to even), on random pairs with exponent gaps up to
    60, exact ties, cancellations and subnormal operands."""
    xs, ys = _bf16_pairs(4000, seed=11)
    got = oracle.add_bf16(xs, ys)
    xf, yf = _f32(xs), _f32(ys)
    exp = np.array([frac_to_bf16_bits(Fraction(float(a)) + Fraction(float(b)))
                    for a, b in zip(xf, yf)], np.uint16)
    assert np.array_equal(got, exp), np.argwhere(got != exp)[:5]
    # the crafted ties really are ties and really round both ways
    t = slice(4000, 4128)
    assert np.any(got[t] == xs[t]) and np.any(got[t] != xs[t])


def test_add_bf16_matches_torch_and_identities():
    xs, ys = _bf16_pairs(20000, seed=12)
    tx = torch.from_numpy(xs.view(np.int16)).view(torch.bfloat16)
    ty = torch.from_numpy(ys.view(np.int16)).view(torch.bfloat16)
    ref = (tx.float() + ty.float()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.add_bf16(xs, ys), ref)
    zero = np.zeros_like(xs)
    assert np.array_equal(oracle.add_bf16(xs, zero), np.where(xs == 0x8000, 0, xs))
    assert np.all(oracle.add_bf16(xs, xs ^ 0x8000) == 0)  # x + (-x) = +0


@pytest.mark.parametrize("group_size", [0, 128])
def test_add_rmsnorm_quant_is_add_then_fused(group_size):
    """The residual form normalizes the new residual stream (the sum), not x:
    it equals the plain fused form applied to torch's bf16 sum, and returns
    that sum as the new residual."""
    x, gamma = synth.rms_inputs(M=24, K=5120, seed=6)
    r = synth.normal_bf16((24, 5120), seed=7, std=2.0)
    q, s, h = oracle.add_rmsnorm_quant(x, r, gamma, 1e-6, group_size)
    hs = (x.float() + r.float()).to(torch.bfloat16)
    assert np.array_equal(h, hs.view(torch.int16).numpy().view(np.uint16))
    if group_size == 0:
        q2, s2 = oracle.rmsnorm_quant(hs, gamma, 1e-6)
    else:
        q2, s2 = oracle.quantize_block(oracle.rmsnorm_bf16(hs, gamma, 1e-6))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    q0, _ = oracle.rmsnorm_quant(x, gamma, 1e-6) if group_size == 0 else (None, None)
    if q0 is not None:
        assert not np.array_equal(q, q0)
