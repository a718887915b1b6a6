"""Pins for the oracle's E4M3FN codec (CPU only).

What fixes the codec, independent of the oracle's own code: the format's
landmark values (tests/golden/e4m3_landmarks.txt, from the OCP FP8 spec), the
structure of the format (127 increasing non-negative finite codes, sign
symmetry), round-trip identity, every midpoint between neighbours, exhaustive
agreement of two independently written encoders on all 2^32 fp32 patterns, and
an exact-rational exhaustive-search encoder on a random sample.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests._exact import nearest_e4m3_exhaustive

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_landmarks.txt")


def _read_golden():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        code, val = line.split()
        rows.append((int(code, 16), val))
    return rows


def test_golden_landmarks_decode():
    for code, val in _read_golden():
        got = oracle.e4m3_decode(code)
        if val == "nan":
            assert math.isnan(got), hex(code)
        else:
            neg = val.startswith("-")
            exp = Fraction(val.lstrip("-"))
            assert Fraction(got) == exp * (-1 if neg else 1), hex(code)
            assert (math.copysign(1.0, got) < 0) == neg, hex(code)


def test_format_structure():
    tab = oracle.decode_table()
    pos = tab[:127]
    assert np.all(np.diff(pos) > 0), "codes 0..126 must increase"
    assert pos[0] == 0.0 and pos[-1] == 448.0
    assert math.isnan(tab[0x7F]) and math.isnan(tab[0xFF])
    for c in range(127):
        assert tab[c | 0x80] == -tab[c]
    assert np.count_nonzero(np.isfinite(tab)) == 254
    # within a binade the step is constant; subnormal step is 2^-9
    assert np.all(np.diff(pos[:9]) == 2.0 ** -9)


def test_encode_decode_identity_all_codes():
    tab = oracle.decode_table()
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        v = tab[c]
        vf = struct.unpack("<f", struct.pack("<f", v))[0]
        assert vf == v
        assert oracle.e4m3_encode(vf) == c, hex(c)
        assert oracle.e4m3_encode_bits(vf) == c, hex(c)


def test_all_midpoints_and_neighbours():
    tab = oracle.decode_table()
    for c in range(126):
        lo, hi = tab[c], tab[c + 1]
        mid = (lo + hi) / 2  # exact: both have <= 4 significant bits
        m32 = np.float32(mid)
        assert float(m32) == mid
        even = c if c % 2 == 0 else c + 1
        below = np.nextafter(m32, np.float32(-1))
        above = np.nextafter(m32, np.float32(1e9))
        for sign in (1, -1):
            sb = 0x80 if sign < 0 else 0
            assert oracle.e4m3_encode(float(sign * m32)) == even | sb
            assert oracle.e4m3_encode(float(sign * below)) == c | sb
            assert oracle.e4m3_encode(float(sign * above)) == (c + 1) | sb


def test_saturation_and_signed_zero():
    for v in (448.0, 448.5, 463.9, 464.0, 1e6, 3.0e38, float("inf")):
        assert oracle.e4m3_encode(v) == 0x7E
        assert oracle.e4m3_encode(-v) == 0xFE
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-30) == 0x80
    assert oracle.e4m3_encode(1e-45) == 0x00  # fp32 subnormal
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00  # tie at half of 2^-9 -> even 0
    assert oracle.e4m3_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01


def test_exact_search_encoder_random_sample():
    tab = oracle.decode_table()
    rng = np.random.default_rng(1234)
    n = 4000
    mags = np.exp2(rng.uniform(-14, 9.2, size=n)).astype(np.float32)
    signs = np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    vals = mags * signs
    got = oracle.e4m3_encode_array(vals)
    for v, g in zip(vals, got):
        assert nearest_e4m3_exhaustive(float(v), tab) == g, float(v)


def test_two_encoders_agree_on_all_fp32_patterns():
    # 2^32 patterns, split in chunks so a failure names a range
    step = 1 << 28
    for lo in range(0, 1 << 32, step):
        assert oracle.encoders_disagree(lo, lo + step) == 0, hex(lo)
