"""Pins for the oracle's scales and quantizers (CPU only).

Fixed independently of the oracle's code by: exact-rational recomputation of
the fp32 scale and of each code (exhaustive search over codes), the invariant
that every nonzero group's largest element encodes to +-448 (over all positive
bf16 amax), the quantize-dequantize error bound, special groups (all zero,
constant magnitude, one nonzero), reductions between granularities (a 1x128
group equals a per-token row of 128; a 128x128 block equals a per-token row of
16384), and for E8M0 the lossless conversion of the page's §1 on every
produced byte plus the golden landmarks.
"""
import os
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import synth
from tests._exact import bf16_all_positive_finite, frac_to_f32, nearest_e4m3_exhaustive

GOLDEN_E8M0 = os.path.join(os.path.dirname(__file__), "golden", "e8m0_landmarks.txt")


def _bits(a_f32: np.ndarray) -> np.ndarray:
    """float32 values that are exact bf16 -> uint16 patterns."""
    u = np.ascontiguousarray(a_f32, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def _f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_scale_is_correctly_rounded_for_every_bf16_amax():
    amax = bf16_all_positive_finite()
    rng = np.random.default_rng(5)
    sample = np.concatenate([amax[:300], amax[-300:], rng.choice(amax, 3000, replace=False)])
    for a in sample:
        s = oracle.scale_f32(float(a))
        assert s == frac_to_f32(Fraction(float(a)) / 448), float(a)


def test_amax_element_encodes_to_max_for_every_bf16_amax():
    amax = bf16_all_positive_finite()
    M = amax.size
    x = np.zeros((M, 128), np.float32)
    x[:, 0] = amax
    x[:, 1] = -amax
    q, s = oracle.quantize_block(_bits(x))
    assert np.all(q[:, 0] == 0x7E)
    assert np.all(q[:, 1] == 0xFE)
    assert np.all(q[:, 2:] == 0)
    r = amax.astype(np.float64) / s.astype(np.float64)[:, 0]
    assert r.min() > 447.0 and r.max() < 449.0


def _random_groups(seed, M=48, K=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K)).astype(np.float32)
    # spread magnitudes across many binades, including tiny and huge rows
    x *= np.exp2(rng.integers(-60, 60, size=(M, 1))).astype(np.float32)
    x[rng.random((M, K)) < 0.05] *= 40.0
    x[rng.random((M, K)) < 0.05] *= 1e-4
    return synth.bf16_bits(synth.to_bf16(x))


def test_block_codes_match_exact_arithmetic():
    tab = oracle.decode_table()
    xb = _random_groups(7, M=6, K=256)
    q, s = oracle.quantize_block(xb)
    xf = _f32(xb)
    for m in range(xb.shape[0]):
        for g in range(2):
            grp = xf[m, 128 * g:128 * g + 128]
            amax = float(np.abs(grp).max())
            s_exact = frac_to_f32(Fraction(amax) / 448)
            assert s[m, g] == s_exact
            for k in range(0, 128, 3):
                v = frac_to_f32(Fraction(float(grp[k])) / Fraction(s_exact))
                assert q[m, 128 * g + k] == nearest_e4m3_exhaustive(v, tab), (m, g, k)


def test_quant_dequant_error_bound():
    tab = oracle.decode_table()
    xb = _random_groups(11, M=64, K=512)
    q, s = oracle.quantize_block(xb)
    x = _f32(xb).astype(np.float64)
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    deq = tab[q] * sf
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.abs(x) / sf))
    e = np.where(np.isfinite(e), e, -6)
    bound = sf * np.exp2(np.maximum(e, -6) - 4) * (1 + 2.0 ** -20) + np.abs(x) * 2.0 ** -23
    assert np.all(np.abs(x - deq) <= bound)


def test_special_groups():
    x = np.zeros((4, 256), np.float32)
    x[0, 128:] = -0.0
    x[0, 130] = 0.0
    x[1, :128] = 3.0
    x[1, 1::2] = -3.0
    x[2, 5] = -(2.0 ** -66)
    x[3, 128:] = np.float32(2.0 ** -133)  # bf16 subnormal, tiny scale
    q, s = oracle.quantize_block(_bits(x))
    assert s[0, 0] == 0.0 and s[0, 1] == 0.0
    assert np.all(q[0, :128] == 0x00)
    exp_neg = np.full(128, 0x80, np.uint8)
    exp_neg[2] = 0x00
    assert np.array_equal(q[0, 128:], exp_neg)
    assert np.all(q[1, 0:128:2] == 0x7E) and np.all(q[1, 1:128:2] == 0xFE)
    assert q[2, 5] == 0xFE and np.count_nonzero(q[2]) == 1
    assert s[3, 1] > 0 and np.all(q[3, 128:] == 0x7E)


def test_token_equals_block_for_one_group_and_weight_block_equals_token_row():
    xb = _random_groups(3, M=40, K=128)
    qb, sb = oracle.quantize_block(xb)
    qt, st = oracle.quantize_token(xb)
    assert np.array_equal(qb, qt) and np.array_equal(sb[:, 0], st)

    w = synth.bf16_bits(synth.weight(256, 384, seed=9))
    qw, sw = oracle.quantize_weight_block(w, fmt=0)
    for i in range(2):
        for j in range(3):
            blk = np.ascontiguousarray(w[128 * i:128 * i + 128, 128 * j:128 * j + 128])
            qr, sr = oracle.quantize_token(blk.reshape(1, -1))
            assert sw[i, j] == sr[0]
            assert np.array_equal(qw[128 * i:128 * i + 128, 128 * j:128 * j + 128].reshape(-1),
                                  qr[0])


def test_token_codes_match_exact_arithmetic():
    tab = oracle.decode_table()
    xb = _random_groups(17, M=4, K=200)
    q, s = oracle.quantize_token(xb)
    xf = _f32(xb)
    for m in range(4):
        s_exact = frac_to_f32(Fraction(float(np.abs(xf[m]).max())) / 448)
        assert s[m] == s_exact
        for k in range(0, 200, 7):
            v = frac_to_f32(Fraction(float(xf[m, k])) / Fraction(s_exact))
            assert q[m, k] == nearest_e4m3_exhaustive(v, tab)


# ---------------------------------------------------------------- E8M0 --
def test_e8m0_golden_landmarks():
    for line in open(GOLDEN_E8M0):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        val, exp = line.split()
        s = np.array([float(Fraction(val))], np.float32)
        codes = oracle.e8m0_lossless(s)
        if exp == "reject":
            assert codes is None, val
        else:
            assert codes is not None and codes[0] == int(exp, 16), val


def test_e8m0_lossless_every_exponent():
    for e in range(-127, 128):
        s = np.array([math.ldexp(1.0, e)], np.float32)
        assert float(s[0]) == math.ldexp(1.0, e)
        codes = oracle.e8m0_lossless(s)
        assert codes is not None and codes[0] == e + 127


def test_e8m0_exponent_is_exact_ceiling():
    rng = np.random.default_rng(21)
    bits = rng.integers(1, 0x7F800000, size=4000, dtype=np.uint32)
    vals = np.concatenate([bits.view(np.float32), np.exp2(np.arange(-149, 128)).astype(np.float32)])
    for v in vals:
        e = oracle.e8m0_exponent(float(v))
        fv = Fraction(float(v))
        if -127 < e < 127:
            assert Fraction(2) ** (e - 1) < fv <= Fraction(2) ** e, float(v)
        elif e == -127:
            assert fv <= Fraction(2) ** -127
    assert oracle.e8m0_exponent(0.0) == -127


def test_e8m0_never_saturates_for_any_bf16_amax():
    amax = bf16_all_positive_finite()
    for a in amax[::1]:
        s = oracle.scale_f32(float(a))
        e = oracle.e8m0_exponent(s)
        assert Fraction(float(a)) <= 448 * Fraction(2) ** e


def test_e8m0_weight_quant_bytes_and_lossless():
    tab = oracle.decode_table()
    w = synth.bf16_bits(synth.weight(256, 256, seed=31))
    w[:128, 128:] = 0  # an all-zero block -> byte 0 and zero codes
    q, s8 = oracle.quantize_weight_block(w, fmt=1)
    q32, s32 = oracle.quantize_weight_block(w, fmt=0)
    assert s8[0, 1] == 0 and np.all(q[:128, 128:] == 0)
    # the byte is the ceiling exponent of the fp32 scale
    for i in range(2):
        for j in range(2):
            assert s8[i, j] == oracle.e8m0_exponent(float(s32[i, j])) + 127
    # every produced scale passes the page's lossless conversion
    p2 = np.ldexp(np.float32(1.0), s8.astype(np.int32) - 127).astype(np.float32)
    codes = oracle.e8m0_lossless(p2)
    assert codes is not None and np.array_equal(codes.reshape(s8.shape), s8)
    # codes: exact division by a power of two, then the E4M3 encoder
    xf = _f32(w).astype(np.float64)
    for (i, j) in ((0, 0), (1, 0), (1, 1)):
        blk = xf[128 * i:128 * i + 128, 128 * j:128 * j + 128]
        sc = math.ldexp(1.0, int(s8[i, j]) - 127)
        for r in range(0, 128, 17):
            for k in range(0, 128, 13):
                v = blk[r, k] / sc
                assert q[128 * i + r, 128 * j + k] == nearest_e4m3_exhaustive(v, tab)


# ------------------------------------------------------- E8M0 1x128 groups --
def test_e8m0_block_codes_match_exact_arithmetic():
    """Byte = ceil(log2(s)) + 127 of the correctly rounded fp32 scale s, found
    with exact rationals; codes = the exhaustive-search nearest E4M3 value of
    the exact quotient x / 2^e."""
    tab = oracle.decode_table()
    xb = _random_groups(23, M=6, K=256)
    q, s8 = oracle.quantize_block_e8m0(xb)
    xf = _f32(xb)
    for m in range(xb.shape[0]):
        for g in range(2):
            grp = xf[m, 128 * g:128 * g + 128]
            s_exact = Fraction(frac_to_f32(Fraction(float(np.abs(grp).max())) / 448))
            e = -127
            while e < 127 and Fraction(2) ** e < s_exact:
                e += 1
            assert s8[m, g] == e + 127, (m, g)
            for k in range(0, 128, 3):
                v = frac_to_f32(Fraction(float(grp[k])) / Fraction(2) ** e)
                assert q[m, 128 * g + k] == nearest_e4m3_exhaustive(v, tab), (m, g, k)


def test_e8m0_block_equals_weight_block_of_repeated_rows():
    """A 1x128 group quantizes like a 128x128 block whose 128 rows are copies
    of it (same amax, so the same byte and the same codes)."""
    xb = _random_groups(29, M=5, K=256)
    q, s8 = oracle.quantize_block_e8m0(xb)
    for m in range(xb.shape[0]):
        w = np.ascontiguousarray(np.repeat(xb[m:m + 1], 128, axis=0))
        qw, sw = oracle.quantize_weight_block(w, fmt=1)
        assert np.array_equal(sw[0], s8[m])
        assert np.all(qw == q[m][None, :])


def test_e8m0_block_zero_group_and_lossless_bytes():
    x = np.zeros((3, 256), np.float32)
    x[0, 128:] = -0.0
    x[1, :] = np.float32(2.0 ** -133)   # bf16 subnormal: byte 0 territory
    x[2, :128] = 1000.0
    x[2, 3] = -1000.0
    q, s8 = oracle.quantize_block_e8m0(_bits(x))
    assert s8[0, 0] == 0 and s8[0, 1] == 0          # e = -127 for amax 0
    assert np.all(q[0, :128] == 0x00) and np.all(q[0, 128:] == 0x80)
    assert s8[2, 0] == 2 + 127                      # s = 1000 / 448 ~ 2.23: 2^1 < s <= 2^2
    assert q[2, 0] == oracle.e4m3_encode(250.0) and q[2, 3] == oracle.e4m3_encode(-250.0)
    assert q[2, 0] == 0x78  # 250 lies nearer 256 than 240
    p2 = np.ldexp(np.float32(1.0), s8.astype(np.int32) - 127).astype(np.float32)
    codes = oracle.e8m0_lossless(p2)
    assert codes is not None and np.array_equal(codes.reshape(s8.shape), s8)


# --------------------------------------------------------------- per-tensor --
def test_tensor_equals_one_row_token_quant_and_exact_scale():
    """One scale for the whole tensor: identical to the per-row quantizer on
    the tensor flattened to a single row; the scale is the correctly rounded
    amax / 448 of all elements and the amax element encodes to +-448."""
    xb = _random_groups(37, M=12, K=384)
    q, s = oracle.quantize_tensor(xb)
    qt, st = oracle.quantize_token(np.ascontiguousarray(xb.reshape(1, -1)))
    assert q.shape == xb.shape
    assert np.array_equal(q.reshape(1, -1), qt) and float(s) == float(st[0])
    xf = _f32(xb)
    amax = float(np.abs(xf).max())
    assert float(s) == frac_to_f32(Fraction(amax) / 448)
    k = int(np.argmax(np.abs(xf).reshape(-1)))
    assert q.reshape(-1)[k] in (0x7E, 0xFE)


def test_tensor_codes_match_exact_arithmetic_and_zero_tensor():
    tab = oracle.decode_table()
    xb = _random_groups(41, M=3, K=256)
    q, s = oracle.quantize_tensor(xb)
    xf = _f32(xb).reshape(-1)
    for k in range(0, xf.size, 7):
        v = frac_to_f32(Fraction(float(xf[k])) / Fraction(float(s)))
        assert q.reshape(-1)[k] == nearest_e4m3_exhaustive(v, tab), k
    z = np.zeros((2, 64), np.float32)
    z[1, 3] = -0.0
    qz, sz = oracle.quantize_tensor(_bits(z))
    assert float(sz) == 0.0 and qz[1, 3] == 0x80 and np.count_nonzero(qz) == 1


def test_gather_quant_indexing():
    """Token gather + 1x128 quantization: identity index is the plain block
    quantizer, a permutation permutes its rows, repeated tokens give equal
    rows, and out-of-range indices give zero rows with zero scales."""
    x = synth.act_col_outliers(12, 384, seed=31)
    q0, s0 = oracle.quantize_block(x)
    q, s = oracle.quantize_block_gather(x, np.arange(12))
    assert np.array_equal(q, q0) and np.array_equal(s, s0)
    perm = np.random.default_rng(32).permutation(12)
    q, s = oracle.quantize_block_gather(x, perm)
    assert np.array_equal(q, q0[perm]) and np.array_equal(s, s0[perm])
    idx = np.array([3, 3, -1, 12, 0, 11, 3])
    q, s = oracle.quantize_block_gather(x, idx)
    assert np.array_equal(q[0], q0[3]) and np.array_equal(q[1], q0[3]) and np.array_equal(q[6], q0[3])
    assert np.all(q[2:4] == 0) and np.all(s[2:4] == 0)
    assert np.array_equal(q[4], q0[0]) and np.array_equal(s[5], s0[11])
