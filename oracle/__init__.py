"""Plain CPU oracle for FP8 (OCP E4M3FN) W8A8 quantization and scaled GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``fp8_w8a8_quantized_amd``) never imports it, and nothing here imports the
product path: the two share no code, headers, tables or helpers.

Layout:
  * ``fp8_oracle.c`` -- the codec, scales, quantizers and RMSNorm as plain C
    (built with gcc, no FMA contraction, no fast-math).
  * this module -- ctypes marshalling for the C part, and the GEMM oracle:
    dequantize each operand to fp64 (code value times its scale, exact in fp64)
    and multiply with an fp64 matrix product, left unrounded.

Pages cited (short tag -> page title, section):
  [FP8-RL]       "FP8-RL: A Practical and Stable Low-Precision Stack for LLM RL",
                 abstract (i): FP8 W8A8 linear layers with blockwise scales, for
                 dense and MoE models.
  [vllm-54894]   "[vllm] [ROCm] DeepSeek V4 ... FP8 WO_A 출력 프로젝션 최적화 분석",
                 §2 (weights viewed as (groups, out, in), scales as
                 (groups, out/128, in/128)), §3 (group-128 activation quant feeding
                 the a8w8 GEMM).
  [sglang-21403] "[sglang] SGLang의 AMD GPU 최적화: RMSNorm과 FP8 Per-token
                 Quantization 커널 융합", §3 (per-token x per-channel a8w8 GEMM
                 with bf16 output, bias None).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libfp8_oracle.so")

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-Wall", "-Wextra", "-shared", "-fPIC"]

GRAN_BLOCK = 0
GRAN_ROW = 1


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc into ``oracle/libfp8_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        f32p = ctypes.POINTER(ctypes.c_float)
        i64 = ctypes.c_int64
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint8
        L.orc_e4m3_encode_bits.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode_bits.restype = ctypes.c_uint8
        L.orc_e4m3_encoders_disagree.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        L.orc_e4m3_encoders_disagree.restype = ctypes.c_uint64
        L.orc_e4m3_encode_array.argtypes = [f32p, i64, u8p]
        L.orc_e4m3_encode_array.restype = None
        L.orc_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_f32.restype = ctypes.c_float
        L.orc_f32_to_bf16_rne.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_rne_array.argtypes = [f32p, i64, u16p]
        L.orc_bf16_rne_array.restype = None
        L.orc_add_bf16.argtypes = [u16p, u16p, i64, u16p]
        L.orc_add_bf16.restype = None
        L.orc_silu_array.argtypes = [u16p, i64, f32p]
        L.orc_silu_array.restype = None
        L.orc_swiglu_bf16.argtypes = [u16p, i64, i64, u16p]
        L.orc_swiglu_bf16.restype = None
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.orc_inverse_rope_bf16.argtypes = [u16p, i64p, f32p, f32p, i64, i64, i64, i64, i64,
                                            u16p]
        L.orc_inverse_rope_bf16.restype = None
        L.orc_scale_f32.argtypes = [ctypes.c_float]
        L.orc_scale_f32.restype = ctypes.c_float
        L.orc_e8m0_exponent.argtypes = [ctypes.c_float]
        L.orc_e8m0_exponent.restype = ctypes.c_int
        L.orc_e8m0_lossless.argtypes = [f32p, i64, u8p]
        L.orc_e8m0_lossless.restype = ctypes.c_int
        L.orc_quantize_block.argtypes = [u16p, i64, i64, u8p, f32p]
        L.orc_quantize_block.restype = None
        L.orc_quantize_block_e8m0.argtypes = [u16p, i64, i64, u8p, u8p]
        L.orc_quantize_block_e8m0.restype = None
        L.orc_quantize_tensor.argtypes = [u16p, i64, u8p, f32p]
        L.orc_quantize_tensor.restype = None
        L.orc_quantize_token.argtypes = [u16p, i64, i64, u8p, f32p]
        L.orc_quantize_token.restype = None
        L.orc_quantize_weight_block.argtypes = [u16p, i64, i64, ctypes.c_int, u8p,
                                                ctypes.c_void_p]
        L.orc_quantize_weight_block.restype = None
        L.orc_rmsnorm_bf16.argtypes = [u16p, u16p, ctypes.c_float, i64, i64, u16p]
        L.orc_rmsnorm_bf16.restype = None
        L.orc_rms_sumsq.argtypes = [u16p, i64]
        L.orc_rms_sumsq.restype = ctypes.c_float
        L.orc_rmsnorm_quant.argtypes = [u16p, u16p, ctypes.c_float, i64, i64, u8p, f32p]
        L.orc_rmsnorm_quant.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _bits16(x) -> np.ndarray:
    """bf16 input as a contiguous uint16 bit-pattern array (numpy or torch CPU)."""
    if isinstance(x, np.ndarray):
        assert x.dtype == np.uint16
        return np.ascontiguousarray(x)
    import torch  # bf16 tensors arrive from the shared input generators

    assert x.dtype == torch.bfloat16 and x.device.type == "cpu"
    return np.ascontiguousarray(x.contiguous().view(torch.int16).numpy().view(np.uint16))


# ---------------------------------------------------------------- codec --
def e4m3_decode(code: int) -> float:
    return lib().orc_e4m3_decode(code)


def e4m3_encode(v: float) -> int:
    return lib().orc_e4m3_encode(v)


def e4m3_encode_bits(v: float) -> int:
    return lib().orc_e4m3_encode_bits(v)


def e4m3_encode_array(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_encode_array(_p(v, ctypes.c_float), v.size, _p(out, ctypes.c_uint8))
    return out


def bf16_rne_array(v: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) of the fp32 values v, round to nearest even."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().orc_bf16_rne_array(_p(v, ctypes.c_float), v.size, _p(out, ctypes.c_uint16))
    return out


def encoders_disagree(lo: int, hi: int) -> int:
    return lib().orc_e4m3_encoders_disagree(lo, hi)


def decode_table() -> np.ndarray:
    """fp64 values of all 256 codes (NaN at 0x7F and 0xFF)."""
    return np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def bf16_to_f32(b: int) -> float:
    return lib().orc_bf16_to_f32(b)


def f32_to_bf16_rne(f: float) -> int:
    return lib().orc_f32_to_bf16_rne(f)


def scale_f32(amax: float) -> float:
    return lib().orc_scale_f32(amax)


def e8m0_exponent(s: float) -> int:
    return lib().orc_e8m0_exponent(s)


def e8m0_lossless(s: np.ndarray):
    """[vllm-54894] §1 lossless conversion; returns codes or None."""
    s = np.ascontiguousarray(s, dtype=np.float32).reshape(-1)
    codes = np.empty(s.shape, np.uint8)
    ok = lib().orc_e8m0_lossless(_p(s, ctypes.c_float), s.size, _p(codes, ctypes.c_uint8))
    return codes if ok else None


# ----------------------------------------------------------- quantizers --
def quantize_block(x):
    """1x128 groups ([FP8-RL] blockwise; [vllm-54894] §3 group size 128)."""
    xb = _bits16(x)
    M, K = xb.shape
    assert K % 128 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.float32)
    lib().orc_quantize_block(_p(xb, ctypes.c_uint16), M, K, _p(q, ctypes.c_uint8),
                             _p(s, ctypes.c_float))
    return q, s


def quantize_block_e8m0(x):
    """1x128 groups with E8M0 scale bytes ([vllm-54894] §1 format, §3 group
    size 128): returns (codes uint8 [M, K], bytes uint8 [M, K/128])."""
    xb = _bits16(x)
    M, K = xb.shape
    assert K % 128 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.uint8)
    lib().orc_quantize_block_e8m0(_p(xb, ctypes.c_uint16), M, K, _p(q, ctypes.c_uint8),
                                  _p(s, ctypes.c_uint8))
    return q, s


def e8m0_value(b: np.ndarray) -> np.ndarray:
    """The power of two an E8M0 byte stands for, 2^(b - 127), as fp64 (exact)."""
    return np.ldexp(1.0, np.asarray(b, dtype=np.int64) - 127)


def quantize_tensor(x):
    """One scale for the whole tensor ([FP8-RL] (ii) KV cache, [E2E-FP8]
    per-tensor dynamic scaling): returns (codes uint8 of x's shape, fp32
    scale as a 0-d array)."""
    xb = _bits16(x)
    flat = np.ascontiguousarray(xb.reshape(-1))
    q = np.empty(flat.shape, np.uint8)
    s = np.empty((), np.float32)
    lib().orc_quantize_tensor(_p(flat, ctypes.c_uint16), flat.size, _p(q, ctypes.c_uint8),
                              s.ctypes.data_as(ctypes.POINTER(ctypes.c_float)))
    return q.reshape(xb.shape), s


def quantize_token(x):
    """One scale per row (per-token activations, per-row weights)."""
    xb = _bits16(x)
    M, K = xb.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((M,), np.float32)
    lib().orc_quantize_token(_p(xb, ctypes.c_uint16), M, K, _p(q, ctypes.c_uint8),
                             _p(s, ctypes.c_float))
    return q, s


def quantize_weight_block(w, fmt: int = 0):
    """128x128 blocks; fmt 0 -> fp32 scales, fmt 1 -> E8M0 bytes."""
    wb = _bits16(w)
    N, K = wb.shape
    assert N % 128 == 0 and K % 128 == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // 128, K // 128), np.float32 if fmt == 0 else np.uint8)
    lib().orc_quantize_weight_block(_p(wb, ctypes.c_uint16), N, K, fmt,
                                    _p(q, ctypes.c_uint8), s.ctypes.data)
    return q, s


def rmsnorm_bf16(x, gamma, eps: float) -> np.ndarray:
    xb, gb = _bits16(x), _bits16(gamma)
    M, K = xb.shape
    y = np.empty((M, K), np.uint16)
    lib().orc_rmsnorm_bf16(_p(xb, ctypes.c_uint16), _p(gb, ctypes.c_uint16), eps, M, K,
                           _p(y, ctypes.c_uint16))
    return y


def rms_sumsq(xrow) -> float:
    xb = _bits16(xrow).reshape(-1)
    return lib().orc_rms_sumsq(_p(xb, ctypes.c_uint16), xb.size)


def rmsnorm_quant(x, gamma, eps: float):
    xb, gb = _bits16(x), _bits16(gamma)
    M, K = xb.shape
    q = np.empty((M, K), np.uint8)
    s = np.empty((M,), np.float32)
    lib().orc_rmsnorm_quant(_p(xb, ctypes.c_uint16), _p(gb, ctypes.c_uint16), eps, M, K,
                            _p(q, ctypes.c_uint8), _p(s, ctypes.c_float))
    return q, s


def add_bf16(x, r) -> np.ndarray:
    """bf16 bits of the residual add: nearest bf16 to the exact x + r."""
    xb, rb = _bits16(x), _bits16(r)
    assert xb.shape == rb.shape
    h = np.empty(xb.shape, np.uint16)
    lib().orc_add_bf16(_p(xb, ctypes.c_uint16), _p(rb, ctypes.c_uint16), xb.size,
                       _p(h, ctypes.c_uint16))
    return h


def add_rmsnorm_quant(x, r, gamma, eps: float, group_size: int = 0):
    """Residual add, then fused RMSNorm + quantization of the sum (the
    add_rmsnorm_quant entry of [sglang-21403] §1).  Returns (q, s, h): codes,
    scales ([M] for group_size 0, [M, K/128] for 128) and h, the new residual
    stream (bf16 bits), which is also what gets normalized."""
    h = add_bf16(x, r)
    if group_size == 0:
        q, s = rmsnorm_quant(h, gamma, eps)
    else:
        q, s = quantize_block(rmsnorm_bf16(h, gamma, eps))
    return q, s, h


def quantize_block_gather(x, row_token):
    """Token gather + 1x128 quantization (the MoE dispatch before the gate_up
    GEMM): row t quantizes x[row_token[t]]; an index outside [0, n_src)
    gives a zero row with zero scales."""
    xb = _bits16(x)
    n_src, K = xb.shape
    idx = np.asarray(row_token, dtype=np.int64)
    valid = (idx >= 0) & (idx < n_src)
    q = np.zeros((idx.size, K), np.uint8)
    s = np.zeros((idx.size, K // 128), np.float32)
    if valid.any():
        qv, sv = quantize_block(np.ascontiguousarray(xb[idx[valid]]))
        q[valid], s[valid] = qv, sv
    return q, s


def inverse_rope_bf16(o, positions, cos_cache, sin_cache, rope_dim: int) -> np.ndarray:
    """bf16 bits [T, H, D] of the inverse RoPE of o (bf16 [T, H, D]) with the
    rotary part in the last rope_dim dims of each head (interleaved pairs)."""
    ob = _bits16(o)
    T, H, D = ob.shape
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    c = np.ascontiguousarray(cos_cache, dtype=np.float32)
    s = np.ascontiguousarray(sin_cache, dtype=np.float32)
    P, half = c.shape
    assert half * 2 == rope_dim and s.shape == c.shape and pos.shape == (T,)
    z = np.empty((T, H, D), np.uint16)
    lib().orc_inverse_rope_bf16(_p(ob, ctypes.c_uint16), _p(pos, ctypes.c_int64),
                                _p(c, ctypes.c_float), _p(s, ctypes.c_float), T, H, D,
                                rope_dim, P, _p(z, ctypes.c_uint16))
    return z


def inverse_rope_group_quant(o, positions, cos_cache, sin_cache, rope_dim: int):
    """Inverse RoPE, then 1x128 E8M0 quantization of each token's flattened
    [H * D] row (feeding the batched MX GEMM): (q [T, H*D], s bytes
    [T, H*D/128], z bits [T, H, D])."""
    z = inverse_rope_bf16(o, positions, cos_cache, sin_cache, rope_dim)
    T = z.shape[0]
    q, s = quantize_block_e8m0(np.ascontiguousarray(z.reshape(T, -1)))
    return q, s, z


def silu_f32(g) -> np.ndarray:
    """SiLU of bf16 values (bits or tensor), correctly rounded to fp32."""
    gb = _bits16(g)
    out = np.empty(gb.shape, np.float32)
    lib().orc_silu_array(_p(gb, ctypes.c_uint16), gb.size, _p(out, ctypes.c_float))
    return out


def swiglu_bf16(gu) -> np.ndarray:
    """bf16 bits [T, I] of bf16_rne(silu(gate) * up), gate = columns [0, I) and
    up = [I, 2I) of the gate_up output gu [T, 2I]."""
    b = _bits16(gu)
    T, I2 = b.shape
    assert I2 % 2 == 0
    y = np.empty((T, I2 // 2), np.uint16)
    lib().orc_swiglu_bf16(_p(b, ctypes.c_uint16), T, I2 // 2, _p(y, ctypes.c_uint16))
    return y


def swiglu_quant(gu):
    """SwiGLU then 1x128 quantization of its bf16 output: (q, s, y)."""
    y = swiglu_bf16(gu)
    q, s = quantize_block(y)
    return q, s, y


# ----------------------------------------------------------------- GEMM --
_DEC = None


def _dec() -> np.ndarray:
    global _DEC
    if _DEC is None:
        _DEC = decode_table()
    return _DEC


def dequant_act(q: np.ndarray, s: np.ndarray, gran: int) -> np.ndarray:
    """fp64 value of each activation element: code value x its scale.
    BLOCK: s[m, k // 128]; ROW: s[m]."""
    d = _dec()[q]
    if gran == GRAN_BLOCK:
        return d * np.repeat(s.astype(np.float64), 128, axis=1)
    return d * s.astype(np.float64)[:, None]


def dequant_weight(q: np.ndarray, s: np.ndarray, gran: int) -> np.ndarray:
    """fp64 value of each weight element.  BLOCK: s[n // 128, k // 128]
    ([vllm-54894] §2 block view); ROW: s[n] (per output channel)."""
    d = _dec()[q]
    if gran == GRAN_BLOCK:
        full = np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)
        return d * full
    return d * s.astype(np.float64)[:, None]


def gemm(qa, qw, sa, sw, gran: int, rows=None) -> np.ndarray:
    """Y[m, n] = sum_k deq(A)[m, k] * deq(W)[n, k] in fp64 (Y = X W^T).

    ``rows`` optionally restricts the output to those rows of A (a sample)."""
    if rows is not None:
        rows = np.asarray(rows)
        qa = qa[rows]
        sa = sa[rows]
    A = dequant_act(qa, sa, gran)
    W = dequant_weight(qw, sw, gran)
    return A @ W.T


def mx_gemm(qa, qw, sa8, sw8, rows=None) -> np.ndarray:
    """Block-scaled GEMM with E8M0 scale bytes ([vllm-54894] §3
    batched_gemm_a8w8_mxscale, one batch): activation bytes sa8 [M, K/128],
    weight bytes sw8 [N/128, K/128]; each byte stands for 2^(b - 127), so this
    is gemm() with those powers of two as the block scales.  fp64."""
    return gemm(qa, qw, e8m0_value(sa8), e8m0_value(sw8), GRAN_BLOCK, rows=rows)


def batched_mx_gemm(qa, qw, sa8, sw8, rows=None) -> np.ndarray:
    """Batched form over groups b ([vllm-54894] §2 weight view (groups, out,
    in), scales (groups, out/128, in/128)): A [M, B, K] with bytes [M, B, K/128],
    W [B, N, K] with bytes [B, N/128, K/128]; Y[m, b, :] = mx_gemm of batch b.
    Returns [len(rows) or M, B, N] fp64."""
    M, B, K = qa.shape
    N = qw.shape[1]
    if rows is None:
        rows = np.arange(M)
    rows = np.asarray(rows)
    out = np.empty((rows.size, B, N), np.float64)
    for b in range(B):
        out[:, b, :] = mx_gemm(np.ascontiguousarray(qa[rows, b, :]), qw[b],
                               np.ascontiguousarray(sa8[rows, b, :]), sw8[b])
    return out


def grouped_gemm(qa, qw, sa, sw, offsets, rows=None) -> np.ndarray:
    """[FP8-RL] MoE coverage: for expert e, rows offsets[e]:offsets[e+1] of A
    use weight qw[e] with block scales sw[e] (BLOCK granularity).  Returns the
    rows listed in ``rows`` (all rows when None), fp64."""
    T = qa.shape[0]
    E = qw.shape[0]
    offsets = np.asarray(offsets, dtype=np.int64)
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows)
    out = np.zeros((rows.size, qw.shape[1]), np.float64)
    expert_of = np.searchsorted(offsets, rows, side="right") - 1
    for e in range(E):
        sel = np.nonzero(expert_of == e)[0]
        if sel.size == 0:
            continue
        out[sel] = gemm(qa[rows[sel]], qw[e], sa[rows[sel]], sw[e], GRAN_BLOCK)
    return out
