"""GPU parity of the quantizers against the CPU oracle: bit-exact E4M3 bytes
and scales (fp32 bits or E8M0 bytes), through the C ABI.

Sizes: small shapes that span several groups/rows with ragged edges, the
special groups (all zero, signed zero, subnormal amax, constant magnitude),
and the full workload sizes (dense linears at M = 8192, the MoE activations,
the rmsnorm workload [4096, 5120], the per-row weight [12288, 5120], the
36-layer policy), each compared in full: every code and every scale.
"""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_amd as fp8
import oracle
import synth
from tests.gpu_util import dev, ensure_library, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _eq_block(xb: torch.Tensor, rows=None):
    q, s = fp8.quantize_block(xb.to(dev()))
    xh = xb if rows is None else xb[torch.as_tensor(rows)]
    oq, os_ = oracle.quantize_block(xh)
    gq, gs = host(q), host(s)
    if rows is not None:
        gq, gs = gq[rows], gs[rows]
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"


def test_block_tiny_linear_input():
    say("quantize_block tiny X [16, 256]")
    X, _ = synth.tiny_linear(seed=0)
    _eq_block(X)


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (37, 384), (64, 4096), (130, 12288),
                                 (5, 640)])
def test_block_shapes(M, K):
    say(f"quantize_block [{M}, {K}]")
    _eq_block(synth.act_col_outliers(M, K, seed=M + K))


def test_block_special_groups():
    say("quantize_block special groups")
    x = np.zeros((6, 512), np.float32)
    x[0, 128:256] = -0.0
    x[1, :128] = 3.0
    x[1, 1:128:2] = -3.0
    x[2, 5] = -(2.0 ** -66)
    x[3, :] = np.float32(2.0 ** -133)           # bf16 subnormal: subnormal fp32 scale
    x[4, :] = np.float32(2.0 ** -70)             # scale below the reciprocal path's bound
    x[4, 7] = np.float32(-(2.0 ** -69))
    x[5, :] = np.float32(3.3895313892515355e38)  # largest bf16
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xt = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    _eq_block(xt)


@pytest.mark.parametrize("M,K", [(8192, 4096), (8192, 12288), (32768, 2048), (32768, 768)])
def test_block_full_size(M, K):
    say(f"quantize_block full [{M}, {K}], every row")
    X = synth.act_col_outliers(M, K, seed=1)
    _eq_block(X)


def _eq_block_e8m0(xb: torch.Tensor, rows=None):
    q, s = fp8.quantize_block_e8m0(xb.to(dev()))
    xh = xb if rows is None else xb[torch.as_tensor(rows)]
    oq, os_ = oracle.quantize_block_e8m0(xh)
    gq, gs = host(q), host(s)
    if rows is not None:
        gq, gs = gq[rows], gs[rows]
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs, os_), f"E8M0 bytes differ at {np.argwhere(gs != os_)[:5]}"


@pytest.mark.parametrize("M,K", [(1, 128), (3, 256), (37, 384), (64, 4096), (130, 12288),
                                 (5, 640)])
def test_block_e8m0_shapes(M, K):
    say(f"quantize_block_e8m0 [{M}, {K}]")
    _eq_block_e8m0(synth.act_col_outliers(M, K, seed=M + K + 1))


def test_block_e8m0_special_groups():
    say("quantize_block_e8m0 special groups")
    x = np.zeros((6, 512), np.float32)
    x[0, 128:256] = -0.0
    x[1, :128] = 3.0
    x[1, 1:128:2] = -3.0
    x[2, 5] = -(2.0 ** -66)
    x[3, :] = np.float32(2.0 ** -133)            # bf16 subnormal amax: byte 0
    x[4, :] = np.float32(448.0 * 2.0 ** 9)       # exact power-of-two scale 2^9
    x[4, 7] = np.float32(-(448.0 * 2.0 ** 9))
    x[5, :] = np.float32(3.3895313892515355e38)  # largest bf16
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    _eq_block_e8m0(torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16))


@pytest.mark.parametrize("M,K", [(8192, 4096), (32768, 768)])
def test_block_e8m0_full_size(M, K):
    say(f"quantize_block_e8m0 full [{M}, {K}], every row")
    X = synth.act_col_outliers(M, K, seed=2)
    _eq_block_e8m0(X)


def _eq_tensors(xs):
    got = fp8.quantize_tensors([x.to(dev()) for x in xs])
    for i, (x, (q, s)) in enumerate(zip(xs, got)):
        oq, os_ = oracle.quantize_tensor(x)
        gq, gs = host(q), host(s)
        assert np.array_equal(gq, oq), f"tensor {i}: codes differ at {np.argwhere(gq != oq)[:5]}"
        assert gs.view(np.uint32)[0] == np.asarray(os_).view(np.uint32), f"tensor {i}: scale"


@pytest.mark.parametrize("shape", [(8,), (1, 2048 * 8), (3, 2048 * 8 + 8), (37, 1000),
                                   (1024, 1024), (5, 7, 128)])
def test_tensor_shapes(shape):
    say(f"quantize_tensors {shape}")
    n = int(np.prod(shape))
    x = synth.act_col_outliers(1, n, seed=n % 97).reshape(shape)
    _eq_tensors([x.contiguous()])


def test_tensor_batch_over_one_launch_and_zero_tensor():
    say("quantize_tensors: 70 tensors (two launch groups) incl. an all-zero one")
    xs = [synth.normal_bf16((16 + 8 * i, 128), seed=300 + i, std=0.5 + i) for i in range(70)]
    xs[5] = torch.zeros((64, 128), dtype=torch.bfloat16)
    _eq_tensors(xs)


def test_tensor_kv_cache_layers():
    say("quantize_tensors: K and V of 4 layers, [8192 tokens, 8 heads x 128]")
    xs = [synth.normal_bf16((8192, 1024), seed=500 + i, std=1.0 + 0.25 * i) for i in range(8)]
    xs[3][17, 5] = 4096.0  # one outlier sets its tensor's scale
    _eq_tensors(xs)


def test_block_deterministic():
    say("quantize_block determinism")
    X = synth.act_col_outliers(512, 4096, seed=3).to(dev())
    q1, s1 = fp8.quantize_block(X)
    q2, s2 = fp8.quantize_block(X)
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


def _eq_token(x: torch.Tensor, rows=None):
    q, s = fp8.quantize_token(x.to(dev()))
    xh = x if rows is None else x[torch.as_tensor(rows)]
    oq, os_ = oracle.quantize_token(xh)
    gq, gs = host(q), host(s)
    if rows is not None:
        gq, gs = gq[rows], gs[rows]
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"


# K = 5120 .. 16384 take one row per 4-wave workgroup (15880: a ragged last
# vector slot); 200 and 20000 the one-wave rows
@pytest.mark.parametrize("M,K", [(1, 8), (5, 200), (33, 4096), (64, 5120), (3, 12288),
                                 (17, 20000), (2, 16384), (3, 15880), (1, 1032)])
def test_token_shapes(M, K):
    say(f"quantize_token [{M}, {K}]")
    _eq_token(synth.act_col_outliers(M, K, seed=M * 7 + K))


def test_token_full_size_weight():
    say("quantize_token full W [12288, 5120], every row")
    W = synth.weight(12288, 5120, seed=5)
    _eq_token(W)


def _eq_rms(h, gamma, group_size, eps=1e-6, rows=None):
    q, s = fp8.rmsnorm_quant(h.to(dev()), gamma.to(dev()), eps, group_size)
    hh = h if rows is None else h[torch.as_tensor(rows)]
    if group_size == 0:
        oq, os_ = oracle.rmsnorm_quant(hh, gamma, eps)
    else:  # fused group variant == RMSNorm -> bf16 -> 1x128 quantization
        y = oracle.rmsnorm_bf16(hh, gamma, eps)
        oq, os_ = oracle.quantize_block(y)
    gq, gs = host(q), host(s)
    if rows is not None:
        gq, gs = gq[rows], gs[rows]
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"


def test_rmsnorm_quant_full_workload():
    say("rmsnorm_quant full [4096, 5120], per token")
    h, gamma = synth.rms_inputs(seed=0)
    _eq_rms(h, gamma, 0)


@pytest.mark.parametrize("M,K,gs", [(3, 8, 0), (7, 200, 0), (5, 4096, 0), (9, 12288, 0),
                                    (4, 40000, 0), (6, 256, 128), (33, 5120, 128),
                                    (3, 40064, 128)])
def test_rmsnorm_quant_shapes(M, K, gs):
    say(f"rmsnorm_quant [{M}, {K}] group_size {gs}")
    h, gamma = synth.rms_inputs(M=M, K=K, seed=M + K)
    _eq_rms(h, gamma, gs)


def test_rmsnorm_quant_group128_full_workload():
    say("rmsnorm_quant full [4096, 5120], group_size 128, every row")
    h, gamma = synth.rms_inputs(seed=1)
    _eq_rms(h, gamma, 128)


def _eq_add_rms(x, r, gamma, group_size, eps=1e-6, rows=None):
    rd = r.to(dev())
    q, s = fp8.add_rmsnorm_quant(x.to(dev()), rd, gamma.to(dev()), eps, group_size)
    if rows is None:
        xh, rh = x, r
    else:
        idx = torch.as_tensor(rows)
        xh, rh = x[idx], r[idx]
    oq, os_, oh = oracle.add_rmsnorm_quant(xh, rh, gamma, eps, group_size)
    gq, gs, gh = host(q), host(s), synth.bf16_bits(rd)
    if rows is not None:
        gq, gs, gh = gq[rows], gs[rows], gh[rows]
    assert np.array_equal(gh, oh), f"residual differs at {np.argwhere(gh != oh)[:5]}"
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"


# with a residual, K = 1032 .. 16384 take one row per 4-wave workgroup
# (15872, 16000: ragged last vector slots)
@pytest.mark.parametrize("M,K,gs", [(3, 8, 0), (7, 200, 0), (5, 4096, 0), (9, 12288, 0),
                                    (4, 40000, 0), (6, 256, 128), (33, 5120, 128),
                                    (3, 40064, 128), (5, 15872, 0), (3, 16000, 128),
                                    (2, 1032, 0), (4, 1152, 128)])
def test_add_rmsnorm_quant_shapes(M, K, gs):
    say(f"add_rmsnorm_quant [{M}, {K}] group_size {gs}")
    x, gamma = synth.rms_inputs(M=M, K=K, seed=M * K + 1)
    r = synth.normal_bf16((M, K), seed=M + 2 * K, std=3.0)
    _eq_add_rms(x, r, gamma, gs)


@pytest.mark.parametrize("gs", [0, 128])
def test_add_rmsnorm_quant_full_workload(gs):
    say(f"add_rmsnorm_quant full [4096, 5120], group_size {gs}")
    x, gamma = synth.rms_inputs(seed=5)
    r = synth.normal_bf16((4096, 5120), seed=6, std=3.0)
    _eq_add_rms(x, r, gamma, gs)


def test_add_rmsnorm_quant_cancelling_residual():
    """r = -x: the new residual is all +0, so every row is the zero row."""
    say("add_rmsnorm_quant with residual -x")
    x, gamma = synth.rms_inputs(M=8, K=4096, seed=9)
    _eq_add_rms(x, -x, gamma, 0)


# ------------------------------------------------------- SwiGLU + 1x128 quant --
def test_silu_all_bf16_patterns():
    """The device silu equals the oracle's correctly rounded silu on every
    bf16 input that is not NaN (bit for bit, signed zeros included)."""
    say("silu of all 65536 bf16 patterns")
    got = host(fp8.silu_f32_of_bf16(0, 1 << 16, device=dev())).view(np.uint32)
    bits = np.arange(1 << 16, dtype=np.uint32)
    keep = ~(((bits & 0x7F80) == 0x7F80) & ((bits & 0x7F) != 0))
    ref = oracle.silu_f32(bits.astype(np.uint16)).view(np.uint32)
    bad = np.nonzero(keep & (got != ref))[0]
    assert bad.size == 0, f"{bad.size} patterns differ, first {bad[:8]}"


def _eq_swiglu(gu, rows=None):
    q, s = fp8.swiglu_quant(gu.to(dev()))
    gh = gu if rows is None else gu[torch.as_tensor(rows)]
    oq, os_, _ = oracle.swiglu_quant(gh)
    gq, gs = host(q), host(s)
    if rows is not None:
        gq, gs = gq[rows], gs[rows]
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("T,I", [(1, 128), (3, 256), (17, 768), (100, 1536), (5, 6144),
                                 (33, 384)])
def test_swiglu_quant_shapes(T, I):
    say(f"swiglu_quant [{T}, 2 x {I}]")
    gu = synth.normal_bf16((T, 2 * I), seed=T * 7 + I, std=3.0)
    _eq_swiglu(gu)


def test_swiglu_quant_every_gate_pattern():
    """Every finite bf16 gate (65280 patterns, in pattern order: some waves'
    gates all lie in the silu table's domain and take the select-free path,
    others hold tiny, large or negative-tail gates), with up values small
    enough that no product overflows; codes and scales bit-exact."""
    say("swiglu_quant over every finite bf16 gate")
    bits = np.arange(1 << 16, dtype=np.uint32)
    g = bits[(bits & 0x7F80) != 0x7F80].astype(np.uint16)
    T, I = 85, 768
    assert g.size == T * I
    gate = torch.from_numpy(g.view(np.int16).reshape(T, I).copy()).view(torch.bfloat16)
    up = (synth.normal_bf16((T, I), seed=5).float() * 1e-3).to(torch.bfloat16)
    _eq_swiglu(torch.cat([gate, up], dim=1))


def test_swiglu_quant_extremes():
    """Gates far in both tails (silu = g, silu = -0), zero groups and
    outlier up values in one tensor."""
    say("swiglu_quant extremes")
    gu = synth.normal_bf16((8, 2 * 256), seed=77, std=2.0)
    gu[0, :256] = 300.0      # silu(g) = g
    gu[1, :256] = -300.0     # silu(g) = -0: a group of signed zeros
    gu[2, 256:] = 0.0        # up = 0
    gu[3, 256 + 5] = 4000.0  # one outlier sets its group's scale
    gu[4, :128] = -80.0      # subnormal silu values
    _eq_swiglu(gu)


def test_swiglu_quant_moe_full_size():
    say("swiglu_quant [32768, 2 x 768], every row")
    gu = synth.normal_bf16((32768, 2 * 768), seed=12, std=2.0)
    _eq_swiglu(gu)


# ------------------------------------------------- token gather + 1x128 quant --
def _eq_gather(x, idx, rows=None):
    q, s = fp8.quantize_block_gather(x.to(dev()), torch.as_tensor(idx, dtype=torch.int32,
                                                                   device=dev()))
    sel = np.arange(len(idx)) if rows is None else rows
    oq, os_ = oracle.quantize_block_gather(x, np.asarray(idx)[sel])
    gq, gs = host(q)[sel], host(s)[sel]
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), "scales differ"


@pytest.mark.parametrize("n_src,K,T", [(1, 128, 1), (7, 256, 30), (100, 2048, 333),
                                       (64, 5120, 17)])
def test_gather_quant_shapes(n_src, K, T):
    say(f"quantize_block_gather x [{n_src}, {K}] -> {T} rows")
    x = synth.act_col_outliers(n_src, K, seed=n_src + K + T)
    idx = np.random.default_rng(T).integers(0, n_src, T)
    _eq_gather(x, idx)


def test_gather_quant_out_of_range_rows_are_zero():
    say("quantize_block_gather with indices outside the token range")
    x = synth.act_col_outliers(10, 256, seed=90)
    _eq_gather(x, np.array([0, -1, 9, 10, 2 ** 31 - 1, -2 ** 31, 5, 5]))


def test_gather_quant_moe_dispatch():
    say("quantize_block_gather: 4096 tokens x 2048 -> 32768 routed rows, every row")
    token_of_row, _ = synth.moe_routing()
    x = synth.normal_bf16((synth.MOE_TOKENS, synth.MOE_HIDDEN), seed=11)
    _eq_gather(x, token_of_row)


# ---------------------------------------- inverse RoPE + 1x128 E8M0 quant --
def _eq_rope(o, pos, cos, sin, groups, rows=None):
    q, s = fp8.inverse_rope_group_quant(o.to(dev()), torch.as_tensor(pos, device=dev()),
                                        torch.as_tensor(cos, device=dev()),
                                        torch.as_tensor(sin, device=dev()), groups)
    T = o.shape[0]
    sel = np.arange(T) if rows is None else rows
    oq, os_, _ = oracle.inverse_rope_group_quant(o[torch.as_tensor(sel)], np.asarray(pos)[sel],
                                                 cos, sin, 2 * cos.shape[1])
    gq = host(q).reshape(T, -1)[sel]
    gs = host(s).reshape(T, -1)[sel]
    assert np.array_equal(gq, oq), f"codes differ at {np.argwhere(gq != oq)[:5]}"
    assert np.array_equal(gs, os_), "E8M0 bytes differ"


@pytest.mark.parametrize("T,H,D,R,G", [(1, 1, 128, 64, 1), (7, 4, 128, 64, 2),
                                       (5, 2, 192, 64, 1),    # groups straddle heads
                                       (9, 8, 64, 64, 4),     # all dims rotary
                                       (3, 4, 128, 0, 1),     # no rotary part
                                       (33, 16, 128, 32, 8)])
def test_inverse_rope_quant_shapes(T, H, D, R, G):
    say(f"inverse_rope_group_quant T={T} H={H} D={D} R={R} groups={G}")
    o, pos = synth.rope_inputs(T, seed=T + H + D + R, heads=H, head_dim=D, seq=11)
    cos, sin = synth.rope_cache(16, R)
    _eq_rope(o, pos, cos, sin, G)


def test_inverse_rope_quant_unaligned_caches_take_scalar_path():
    """cos/sin starting 4 bytes into an allocation cannot take 16-byte loads;
    the result is the same."""
    say("inverse_rope_group_quant with 4-byte aligned cos/sin")
    o, pos = synth.rope_inputs(5, seed=47, heads=4, head_dim=128, seq=9)
    cos, sin = synth.rope_cache(16, 64)
    cb = torch.zeros(cos.size + 1, dtype=torch.float32, device=dev())
    sb = torch.zeros(sin.size + 1, dtype=torch.float32, device=dev())
    cb[1:] = torch.as_tensor(cos.reshape(-1), device=dev())
    sb[1:] = torch.as_tensor(sin.reshape(-1), device=dev())
    cv, sv = cb[1:].view(16, 32), sb[1:].view(16, 32)
    q, s = fp8.inverse_rope_group_quant(o.to(dev()), torch.as_tensor(pos, device=dev()), cv, sv, 2)
    oq, os_, _ = oracle.inverse_rope_group_quant(o, pos, cos, sin, 64)
    assert np.array_equal(host(q).reshape(5, -1), oq)
    assert np.array_equal(host(s).reshape(5, -1), os_)


def test_inverse_rope_quant_out_of_range_positions():
    say("inverse_rope_group_quant with positions outside the cache")
    o, _ = synth.rope_inputs(6, seed=41, heads=4, head_dim=128)
    cos, sin = synth.rope_cache(16, 64)
    _eq_rope(o, np.array([0, 16, -1, 15, 2 ** 40, 3], np.int64), cos, sin, 2)


def test_inverse_rope_quant_full_workload():
    T = 8192
    say(f"inverse_rope_group_quant [{T}, 64, 128], R = 64, 8 groups, every row")
    o, pos = synth.rope_inputs(T, seed=42)
    cos, sin = synth.rope_cache()
    _eq_rope(o, pos, cos, sin, synth.ROPE_GROUPS)


def _eq_req(ws, fmt, out=None, block_rows=None):
    res = fp8.requantize_weights([w.to(dev()) if not w.is_cuda else w for w in ws], fmt)
    for i, (w, (q, s)) in enumerate(zip(ws, res)):
        if block_rows is None:
            wh = w.cpu()
            gq, gs = host(q), host(s)
        else:
            br = block_rows[i]
            wh = w[br * 128:(br + 1) * 128].cpu()
            gq = host(q[br * 128:(br + 1) * 128])
            gs = host(s[br:br + 1])
        oq, os_ = oracle.quantize_weight_block(wh, fmt)
        assert np.array_equal(gq, oq), f"weight {i}: codes differ at {np.argwhere(gq != oq)[:5]}"
        if fmt == 0:
            assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"weight {i} scales"
        else:
            assert np.array_equal(gs, os_), f"weight {i} E8M0 bytes"
            p2 = np.ldexp(np.float32(1.0), gs.astype(np.int32) - 127).astype(np.float32)
            codes = oracle.e8m0_lossless(p2)
            assert codes is not None and np.array_equal(codes.reshape(gs.shape), gs)


@pytest.mark.parametrize("fmt", [0, 1])
def test_requant_small_batch(fmt):
    say(f"requantize_weights small batch fmt {fmt}")
    _, W0 = synth.tiny_linear(seed=0)
    ws = [W0, synth.weight(384, 640, seed=2), synth.weight(128, 128, seed=3),
          synth.weight(1536 * 3, 2048, seed=4)]  # last: three stacked experts
    z = torch.zeros((256, 256), dtype=torch.bfloat16)
    z[128:, :128] = 1e-30
    ws.append(z)
    _eq_req(ws, fmt)


def test_requant_more_descriptors_than_one_launch():
    say("requantize_weights 70 descriptors")
    ws = [synth.weight(128, 128 * (1 + i % 3), seed=100 + i) for i in range(70)]
    _eq_req(ws, 0)
    _eq_req(ws, 1)


@pytest.mark.parametrize("part", range(4))
@pytest.mark.parametrize("fmt", [0, 1])
def test_requant_full_policy(fmt, part):
    """The whole 36-layer policy (144 weights, 6.9e9 elements) in one call;
    each part compares every code and scale of 9 layers' weights (36
    tensors) against the oracle, so the four parts cover all 144."""
    say(f"requantize_weights full 36-layer policy fmt {fmt}, layers {9 * part}..{9 * part + 8}"
        ", every block")
    ws = []
    for layer in range(synth.POLICY_LAYERS):
        for j, (name, (N, K)) in enumerate(synth.DENSE_SHAPES.items()):
            ws.append(synth.weight(N, K, seed=1000 + 4 * layer + j, device=dev()))
    res = fp8.requantize_weights(ws, fmt)
    torch.cuda.synchronize()
    for i in range(36 * part, 36 * (part + 1)):
        oq, os_ = oracle.quantize_weight_block(ws[i].cpu(), fmt)
        q, s = res[i]
        gq = host(q)
        assert np.array_equal(gq, oq), f"tensor {i}: codes differ at {np.argwhere(gq != oq)[:5]}"
        gs = host(s)
        if fmt == 0:
            assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32)), f"tensor {i} scales"
        else:
            assert np.array_equal(gs, os_), f"tensor {i} E8M0 bytes"
        del oq, os_, gq
    del ws, res
    torch.cuda.empty_cache()


def test_error_leaves_outputs_untouched():
    say("error paths leave outputs untouched")
    L = fp8.load_library()
    x = torch.ones((4, 200), dtype=torch.bfloat16, device=dev())
    q = torch.full((4, 200), 0xAB, dtype=torch.uint8, device=dev())
    s = torch.full((4, 2), 7.0, dtype=torch.float32, device=dev())
    import ctypes

    rc = L.fp8_quantize_block(ctypes.c_void_p(x.data_ptr()), 4, 200, ctypes.c_void_p(q.data_ptr()),
                              ctypes.c_void_p(s.data_ptr()), None)
    assert rc == -2
    assert torch.all(q == 0xAB) and torch.all(s == 7.0)


def test_forced_foreign_arch_is_refused(monkeypatch):
    say("FP8W8A8_FORCE_ARCH refusal")
    monkeypatch.setenv("FP8W8A8_FORCE_ARCH", "gfx942")
    x = torch.ones((4, 128), dtype=torch.bfloat16, device=dev())
    with pytest.raises(fp8.Fp8Error) as ei:
        fp8.quantize_block(x)
    assert ei.value.status == -4


# ------------------------------------------------------------ seeded sweeps --
def test_quantizer_shape_sweep():
    """Seeded shapes through every quantizer, each bit-exact against the
    oracle: rows 1..3000 with the 64- and 256-row edges mixed in, K a multiple
    of 128 up to 6144 (RMSNorm forms: any K up to 6144, multiples of 8 for
    the per-token form), SwiGLU widths up to 3072, gathers with repeated and
    unsorted source rows."""
    rng = np.random.default_rng(31)
    edges = [1, 63, 64, 65, 255, 256, 257]
    for i in range(10):
        M = edges[i] if i < len(edges) else int(rng.integers(1, 3001))
        K = 128 * int(rng.integers(1, 49))
        say(f"quantizer sweep {i}: M={M} K={K}")
        x = synth.act_col_outliers(M, K, seed=5000 + i)
        _eq_block(x)
        _eq_block_e8m0(x)
        _eq_token(x)
        h, gamma = synth.rms_inputs(M=M, K=K, seed=6000 + i)
        _eq_rms(h, gamma, 128)
        Kr = 8 * int(rng.integers(1, 769))
        h2, gamma2 = synth.rms_inputs(M=M, K=Kr, seed=7000 + i)
        say(f"quantizer sweep {i}: rmsnorm per token K={Kr}")
        _eq_rms(h2, gamma2, 0)
        _eq_add_rms(h2, synth.normal_bf16((M, Kr), seed=8000 + i, std=3.0), gamma2, 0)
        I = 128 * int(rng.integers(1, 25))
        say(f"quantizer sweep {i}: swiglu I={I}, gather")
        _eq_swiglu(synth.normal_bf16((M, 2 * I), seed=9000 + i, std=3.0))
        n_src = int(rng.integers(1, 400))
        _eq_gather(synth.normal_bf16((n_src, K), seed=9500 + i), rng.integers(0, n_src, size=M))
