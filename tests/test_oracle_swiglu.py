"""Pins for the oracle's SiLU and SwiGLU (the MoE chain between the gate_up and
down grouped GEMMs).

SiLU of a bf16 input is defined as the fp32 value nearest to g / (1 + e^-g).
It is pinned on every finite bf16 input: against 60-digit decimal arithmetic
where |g| < 200, and against closed forms outside (the value rounds to g above,
to -0 below).  SwiGLU is pinned by closed forms that fail if gate and up are
swapped or the product is taken in another precision, and by torch's SiLU in
fp64 to one bf16 ulp.
"""
import decimal
from fractions import Fraction

import numpy as np
import torch

import oracle
import synth
from _exact import frac_to_f32


def _all_finite_bf16():
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]  # drop Inf and NaN
    return b.astype(np.uint16)


def test_silu_correctly_rounded_on_every_bf16():
    bits = _all_finite_bf16()
    got = oracle.silu_f32(bits)
    g = (bits.astype(np.uint32) << 16).view(np.float32)
    ctx = decimal.Context(prec=60, Emax=10 ** 6, Emin=-10 ** 6)
    exp = np.empty_like(got)
    for i, v in enumerate(g.tolist()):
        if v == 0.0:
            exp[i] = v  # silu(+-0) = +-0
        elif v >= 200.0:
            exp[i] = v  # g * sigmoid(g) within e^-200 of g: rounds to g
        elif v <= -200.0:
            exp[i] = -0.0  # |g e^g| < 2^-150: rounds to -0
        else:
            d = ctx.divide(decimal.Decimal(v), ctx.add(1, ctx.exp(decimal.Decimal(-v))))
            exp[i] = frac_to_f32(Fraction(d))
            if exp[i] == 0.0 and v < 0:
                exp[i] = -0.0
    gi, ei = got.view(np.uint32), exp.view(np.uint32)
    bad = np.nonzero(gi != ei)[0]
    assert bad.size == 0, [(float(g[i]), float(got[i]), float(exp[i])) for i in bad[:5]]


def test_silu_landmarks():
    one = np.array([0x3F80], np.uint16)  # 1.0: 1 / (1 + 1/e)
    assert oracle.silu_f32(one)[0] == np.float32(0.7310585786300049)
    assert oracle.silu_f32(np.array([0x8000], np.uint16)).view(np.uint32)[0] == 0x80000000


def test_swiglu_closed_forms_and_half_order():
    T, I = 5, 256
    up = synth.normal_bf16((T, I), seed=4)
    # gate = 20 (silu(20) rounds to 20 in fp32): y = bf16(20 * up)
    gate = torch.full((T, I), 20.0, dtype=torch.bfloat16)
    y = oracle.swiglu_bf16(torch.cat([gate, up], dim=1))
    ref = (up.float() * 20.0).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)
    # up = 1: y = bf16(silu(gate)); swapping the halves would give silu(1) * gate
    g2 = synth.normal_bf16((T, I), seed=5, std=4.0)
    y2 = oracle.swiglu_bf16(torch.cat([g2, torch.ones((T, I), dtype=torch.bfloat16)], dim=1))
    s = oracle.silu_f32(g2)
    ref2 = torch.from_numpy(s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y2, ref2)
    # gate = -300: silu = -0, so y = -0 * up: signed zeros
    g3 = torch.full((T, I), -300.0, dtype=torch.bfloat16)
    y3 = oracle.swiglu_bf16(torch.cat([g3, up], dim=1))
    assert np.all((y3 & 0x7FFF) == 0)


def test_swiglu_within_one_bf16_ulp_of_torch_fp64():
    gu = synth.normal_bf16((64, 2 * 768), seed=8, std=2.0)
    y = oracle.swiglu_bf16(gu).astype(np.int32)
    g, u = gu[:, :768].double(), gu[:, 768:].double()
    ref = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
    rb = ref.view(torch.int16).numpy().view(np.uint16).astype(np.int32)
    assert np.all(np.abs(y - rb) <= 1)
    assert np.mean(y == rb) > 0.99


def test_swiglu_quant_is_swiglu_then_block_quant():
    gu = synth.normal_bf16((6, 2 * 384), seed=9, std=3.0)
    q, s, y = oracle.swiglu_quant(gu)
    q2, s2 = oracle.quantize_block(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
