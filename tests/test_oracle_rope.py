"""Pins for the oracle's inverse RoPE (ahead of the E8M0 group quantization
that feeds the batched MX GEMM).

Pinned by: angle 0 is the identity; a quarter turn moves each pair (y0, y1)
to (y1, -y0), which fixes the pairing (interleaved, last R dims) and the sign;
rotating the result forward in fp64 gives back the input within bf16
rounding; exact rational arithmetic for the per-operation fp32 rounding; the
pass-through dims; the zero row of an out-of-range position; and the group
quantization being the E8M0 1x128 quantizer of the flattened row.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth
from _exact import frac_to_bf16_bits, frac_to_f32

T, H, D, R = 6, 4, 128, 64


def _caches(P, angle):
    c = np.full((P, R // 2), np.float32(np.cos(angle)), np.float32)
    s = np.full((P, R // 2), np.float32(np.sin(angle)), np.float32)
    return c, s


def _f(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32)


def test_angle_zero_is_identity():
    o, _ = synth.rope_inputs(T, seed=1, heads=H, head_dim=D)
    c = np.ones((4, R // 2), np.float32)
    s = np.zeros((4, R // 2), np.float32)
    z = oracle.inverse_rope_bf16(o, np.zeros(T, np.int64), c, s, R)
    assert np.array_equal(z, synth.bf16_bits(o))


def test_quarter_turn_fixes_pairing_and_sign():
    o, _ = synth.rope_inputs(T, seed=2, heads=H, head_dim=D)
    c = np.zeros((4, R // 2), np.float32)
    s = np.ones((4, R // 2), np.float32)
    z = _f(oracle.inverse_rope_bf16(o, np.full(T, 3, np.int64), c, s, R))
    y = o.float().numpy()
    rot = y[..., D - R:]
    assert np.array_equal(z[..., :D - R], y[..., :D - R])
    assert np.array_equal(z[..., D - R::2], rot[..., 1::2])       # x0 = y1
    assert np.array_equal(z[..., D - R + 1::2], -rot[..., 0::2])  # x1 = -y0


def test_forward_rotation_recovers_input():
    o, pos = synth.rope_inputs(64, seed=3, heads=H, head_dim=D, seq=40)
    c, s = synth.rope_cache(64, R)
    z = _f(oracle.inverse_rope_bf16(o, pos, c, s, R)).astype(np.float64)
    cc, ss = c[pos].astype(np.float64)[:, None, :], s[pos].astype(np.float64)[:, None, :]
    x0, x1 = z[..., D - R::2], z[..., D - R + 1::2]
    f0 = x0 * cc - x1 * ss   # forward rotation by the same angle
    f1 = x0 * ss + x1 * cc
    y = o.double().numpy()
    nrm = np.sqrt(y[..., D - R::2] ** 2 + y[..., D - R + 1::2] ** 2)
    bound = 2 ** -7 * nrm + 1e-30  # two bf16 roundings of values within the pair norm
    assert np.all(np.abs(f0 - y[..., D - R::2]) <= bound)
    assert np.all(np.abs(f1 - y[..., D - R + 1::2]) <= bound)


def test_exact_per_operation_rounding():
    o, pos = synth.rope_inputs(3, seed=4, heads=2, head_dim=D, seq=3)
    c, s = synth.rope_cache(8, R)
    z = oracle.inverse_rope_bf16(o, pos, c, s, R)
    y = o.float().numpy()
    for t in range(3):
        for h in range(2):
            for i in range(R // 2):
                y0, y1 = float(y[t, h, D - R + 2 * i]), float(y[t, h, D - R + 2 * i + 1])
                cf, sf = float(c[pos[t], i]), float(s[pos[t], i])
                a = frac_to_f32(Fraction(y0) * Fraction(cf))
                b = frac_to_f32(Fraction(y1) * Fraction(sf))
                x0 = frac_to_f32(Fraction(a) + Fraction(b))
                a1 = frac_to_f32(Fraction(y1) * Fraction(cf))
                b1 = frac_to_f32(Fraction(y0) * Fraction(sf))
                x1 = frac_to_f32(Fraction(a1) - Fraction(b1))
                assert z[t, h, D - R + 2 * i] == frac_to_bf16_bits(Fraction(x0)) | (
                    0x8000 if (x0 == 0 and np.signbit(x0)) else 0)
                assert z[t, h, D - R + 2 * i + 1] == frac_to_bf16_bits(Fraction(x1)) | (
                    0x8000 if (x1 == 0 and np.signbit(x1)) else 0)


def test_out_of_range_position_zero_row():
    o, _ = synth.rope_inputs(4, seed=5, heads=H, head_dim=D)
    c, s = synth.rope_cache(16, R)
    z = oracle.inverse_rope_bf16(o, np.array([0, 16, -1, 15]), c, s, R)
    assert np.all(z[1] == 0) and np.all(z[2] == 0)
    assert np.any(z[0] != 0) and np.any(z[3] != 0)


def test_group_quant_is_e8m0_block_of_flattened_rows():
    o, pos = synth.rope_inputs(5, seed=6, heads=H, head_dim=D)
    c, s = synth.rope_cache(64, R)
    q, sc, z = oracle.inverse_rope_group_quant(o, pos, c, s, R)
    q2, s2 = oracle.quantize_block_e8m0(np.ascontiguousarray(z.reshape(5, -1)))
    assert np.array_equal(q, q2) and np.array_equal(sc, s2)
    assert q.shape == (5, H * D) and sc.shape == (5, H * D // 128)
