"""MI355X (gfx950) FP8 W8A8 quantization and scaled GEMM.

Thin Python binding over the C ABI of ``libfp8w8a8.so`` (include/fp8w8a8.h).
Every function here only checks tensor properties, allocates outputs with
torch on the input's device and passes raw pointers plus torch's current HIP
stream to the library; all computation runs in the library's HIP kernels.
If the library has not been built, every call raises ``Fp8LibraryMissing``.

The pairs returned by the quantizers are the (fp8 tensor, scale) tuples that
the page "[sglang] SGLang의 AMD GPU 최적화: RMSNorm과 FP8 Per-token Quantization
커널 융합" (§3) passes straight into the GEMM without re-quantizing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Sequence, Tuple

import torch

__all__ = [
    "Fp8Error", "Fp8LibraryMissing", "GRAN_BLOCK", "GRAN_ROW", "SCALE_F32", "SCALE_E8M0",
    "quantize_tensors", "quantize_tensor", "quantize_block_e8m0", "batched_gemm_a8w8_mxscale",
    "library_path", "load_library", "quantize_block", "quantize_token", "rmsnorm_quant",
    "add_rmsnorm_quant", "swiglu_quant", "quantize_block_gather", "inverse_rope_group_quant",
    "silu_f32_of_bf16", "requantize_weights", "gemm_a8w8_scaled", "gemm_workspace_size",
    "batched_gemm_mxscale_workspace_size", "grouped_gemm_a8w8_scaled", "encode_f32_bits",
    "status_string", "abi_version",
]

GRAN_BLOCK, GRAN_ROW = 0, 1
SCALE_F32, SCALE_E8M0 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libfp8w8a8.so")


class Fp8Error(RuntimeError):
    """A library call returned a non-OK status."""

    def __init__(self, func: str, status: int, message: str):
        super().__init__(f"{func}: status {status} ({message})")
        self.status = status


class Fp8LibraryMissing(RuntimeError):
    """libfp8w8a8.so has not been built."""


class _WeightDesc(ctypes.Structure):
    _fields_ = [("w_bf16", ctypes.c_void_p), ("q_e4m3", ctypes.c_void_p),
                ("s", ctypes.c_void_p), ("N", ctypes.c_int64), ("K", ctypes.c_int64)]


class _TensorDesc(ctypes.Structure):
    _fields_ = [("x_bf16", ctypes.c_void_p), ("q_e4m3", ctypes.c_void_p),
                ("s", ctypes.c_void_p), ("n", ctypes.c_int64)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libfp8w8a8.so (once) and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise Fp8LibraryMissing(
            f"{_LIB_PATH} is not built; run fp8_w8a8_quantized_amd/build.py "
            "(or __graft_entry__.build())")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sz = ctypes.c_size_t
    sig = {
        "fp8_abi_version": ([], i32),
        "fp8_status_string": ([i32], ctypes.c_char_p),
        "fp8_build_source_hash": ([], ctypes.c_char_p),
        "fp8_quantize_block": ([vp, i64, i64, vp, vp, vp], i32),
        "fp8_quantize_block_e8m0": ([vp, i64, i64, vp, vp, vp], i32),
        "fp8_quantize_token": ([vp, i64, i64, vp, vp, vp], i32),
        "fp8_batched_gemm_a8w8_mxscale": ([vp, vp, vp, vp, vp, i64, i64, i64, i64, vp, sz, vp],
                                          i32),
        "fp8_batched_gemm_mxscale_workspace_size": ([i64, i64, i64, i64], sz),
        "fp8_rmsnorm_quant": ([vp, vp, vp, vp, f32, i64, i64, i32, vp], i32),
        "fp8_add_rmsnorm_quant": ([vp, vp, vp, vp, vp, f32, i64, i64, i32, vp], i32),
        "fp8_swiglu_quant": ([vp, i64, i64, vp, vp, vp], i32),
        "fp8_quantize_block_gather": ([vp, i64, i64, vp, i64, vp, vp, vp], i32),
        "fp8_inverse_rope_group_quant": ([vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, vp, vp,
                                          vp], i32),
        "fp8_silu_f32_of_bf16": ([ctypes.c_uint32, i64, vp, vp], i32),
        "fp8_mfma_rate_probe": ([i64, vp, vp], i32),
        "fp8_requantize_workspace_size": ([i32], sz),
        "fp8_requantize_weights": ([ctypes.POINTER(_WeightDesc), i32, i32, vp, sz, vp], i32),
        "fp8_gemm_a8w8_scaled": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp], i32),
        "fp8_gemm_workspace_size": ([i64, i64, i64, i32], sz),
        "fp8_gemm_a8w8_scaled_noalloc": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp], i32),
        "fp8_grouped_gemm_a8w8_scaled": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, vp], i32),
        "fp8_quantize_tensors": ([ctypes.POINTER(_TensorDesc), i32, vp], i32),
        "fp8_encode_f32_bits": ([ctypes.c_uint64, i64, vp, vp], i32),
        "fp8_bf16_round_f32_bits": ([ctypes.c_uint64, i64, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def status_string(status: int) -> str:
    return load_library().fp8_status_string(status).decode()


def abi_version() -> int:
    return load_library().fp8_abi_version()


def _check(func: str, rc: int) -> None:
    if rc != 0:
        raise Fp8Error(func, rc, status_string(rc))


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t: torch.Tensor, dtype, ndim: int, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(t: torch.Tensor, name: str) -> None:
    """The last check before a library call (every buffer is on t's device)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a HIP device")


def _need_buf(t, dtypes, shape, name: str, device) -> None:
    """A buffer the library reads or writes by raw pointer: its dtype, exact
    shape, contiguity and device are checked before any call, so a wrong
    buffer is a Python error rather than an out-of-bounds device access."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be one of {dtypes}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


_CODES = (torch.uint8, torch.float8_e4m3fn)
_F32 = (torch.float32,)
_U8 = (torch.uint8,)
_BF16 = (torch.bfloat16,)


def _out_pair(out, q_shape, s_dtype, s_shape, device):
    """Checked (q, s) output buffers from ``out``, or new ones."""
    if out is None:
        return (torch.empty(q_shape, dtype=torch.uint8, device=device),
                torch.empty(s_shape, dtype=s_dtype, device=device))
    q, s = out
    _need_buf(q, _CODES, q_shape, "out[0]", device)
    _need_buf(s, (s_dtype,), s_shape, "out[1]", device)
    return q.view(torch.uint8), s


# ------------------------------------------------------------ quantizers --
def quantize_block(x: torch.Tensor, out=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 [M, K] -> (E4M3 bytes uint8 [M, K], fp32 scales [M, K/128]).
    ``out`` may supply the (q, s) buffers."""
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    q, s = _out_pair(out, (M, K), torch.float32, (M, K // 128), x.device)
    _on_gpu(x, "x")
    L = load_library()
    _check("fp8_quantize_block", L.fp8_quantize_block(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def quantize_block_e8m0(x: torch.Tensor, out=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 [M, K] -> (E4M3 bytes uint8 [M, K], E8M0 scale bytes uint8 [M, K/128]).
    ``out`` may supply the (q, s) buffers."""
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    q, s = _out_pair(out, (M, K), torch.uint8, (M, K // 128), x.device)
    _on_gpu(x, "x")
    L = load_library()
    _check("fp8_quantize_block_e8m0",
           L.fp8_quantize_block_e8m0(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def quantize_token(x: torch.Tensor, out=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 [M, K] -> (E4M3 bytes uint8 [M, K], fp32 scales [M]).
    ``out`` may supply the (q, s) buffers."""
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    q, s = _out_pair(out, (M, K), torch.float32, (M,), x.device)
    _on_gpu(x, "x")
    L = load_library()
    _check("fp8_quantize_token", L.fp8_quantize_token(_ptr(x), M, K, _ptr(q), _ptr(s), _stream(x)))
    return q, s


def _rms_scale_shape(M: int, K: int, group_size: int):
    return (M,) if group_size == 0 else (M, K // 128)


def rmsnorm_quant(x: torch.Tensor, gamma: torch.Tensor, eps: float = 1e-6,
                  group_size: int = 0, out=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fused RMSNorm + FP8 quantization.  group_size 0: scales [M];
    group_size 128: scales [M, K/128].  ``out`` may supply the (q, s) buffers."""
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    _need_buf(gamma, _BF16, (K,), "gamma", x.device)
    q, s = _out_pair(out, (M, K), torch.float32, _rms_scale_shape(M, K, group_size), x.device)
    _on_gpu(x, "x")
    L = load_library()
    _check("fp8_rmsnorm_quant", L.fp8_rmsnorm_quant(_ptr(q), _ptr(x), _ptr(s), _ptr(gamma),
                                                   float(eps), M, K, group_size, _stream(x)))
    return q, s


def add_rmsnorm_quant(x: torch.Tensor, residual: torch.Tensor, gamma: torch.Tensor,
                      eps: float = 1e-6, group_size: int = 0, out=None
                      ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Residual add + fused RMSNorm + FP8 quantization.  ``residual`` is
    updated in place to bf16(x + residual), which is then normalized and
    quantized as in ``rmsnorm_quant``.  Returns (q, s)."""
    _need(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    _need_buf(residual, _BF16, (M, K), "residual", x.device)
    _need_buf(gamma, _BF16, (K,), "gamma", x.device)
    q, s = _out_pair(out, (M, K), torch.float32, _rms_scale_shape(M, K, group_size), x.device)
    _on_gpu(x, "x")
    L = load_library()
    _check("fp8_add_rmsnorm_quant",
           L.fp8_add_rmsnorm_quant(_ptr(q), _ptr(x), _ptr(residual), _ptr(s), _ptr(gamma),
                                   float(eps), M, K, group_size, _stream(x)))
    return q, s


def swiglu_quant(gu: torch.Tensor, out=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """SwiGLU of the gate_up output gu bf16 [T, 2I] (gate first), then 1x128
    quantization: codes [T, I] and scales [T, I/128]."""
    _need(gu, torch.bfloat16, 2, "gu")
    T, I2 = gu.shape
    if I2 % 2:
        raise ValueError("gu must have an even number of columns")
    I = I2 // 2
    q, s = _out_pair(out, (T, I), torch.float32, (T, I // 128), gu.device)
    _on_gpu(gu, "gu")
    L = load_library()
    _check("fp8_swiglu_quant", L.fp8_swiglu_quant(_ptr(gu), T, I, _ptr(q), _ptr(s), _stream(gu)))
    return q, s


def quantize_block_gather(x: torch.Tensor, row_token: torch.Tensor, out=None
                          ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Token gather + 1x128 quantization: row t of the result quantizes
    x[row_token[t]] (x bf16 [n_src, K], row_token int32 [T] on the device)."""
    _need(x, torch.bfloat16, 2, "x")
    _need(row_token, torch.int32, 1, "row_token")
    n_src, K = x.shape
    T = row_token.shape[0]
    if row_token.device != x.device:
        raise ValueError("row_token must be on x's device")
    q, s = _out_pair(out, (T, K), torch.float32, (T, K // 128), x.device)
    _on_gpu(x, "x")
    L = load_library()
    _check("fp8_quantize_block_gather",
           L.fp8_quantize_block_gather(_ptr(x), n_src, K, _ptr(row_token), T, _ptr(q), _ptr(s),
                                       _stream(x)))
    return q, s


def inverse_rope_group_quant(o: torch.Tensor, positions: torch.Tensor, cos_cache: torch.Tensor,
                             sin_cache: torch.Tensor, num_groups: int, out=None
                             ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Inverse RoPE of o bf16 [T, H, D] (rotary part: the last 2 * cos_cache.shape[1]
    dims of each head, interleaved pairs), then 1x128 E8M0 quantization.
    Returns (codes [T, G, H*D/G], E8M0 bytes [T, G, H*D/(128 G)]) with G =
    num_groups, the token-major layout batched_gemm_a8w8_mxscale takes."""
    _need(o, torch.bfloat16, 3, "o")
    T, H, D = o.shape
    _need(cos_cache, torch.float32, 2, "cos_cache")
    P, half = cos_cache.shape
    _need_buf(positions, (torch.int64,), (T,), "positions", o.device)
    _need_buf(cos_cache, _F32, (P, half), "cos_cache", o.device)
    _need_buf(sin_cache, _F32, (P, half), "sin_cache", o.device)
    G = int(num_groups)
    if G <= 0 or H % G:
        raise ValueError(f"num_groups must be positive and divide H = {H}, got {G}")
    Kg = H * D // G
    q, s = _out_pair(out, (T, G, Kg), torch.uint8, (T, G, Kg // 128), o.device)
    _on_gpu(o, "o")
    L = load_library()
    _check("fp8_inverse_rope_group_quant",
           L.fp8_inverse_rope_group_quant(_ptr(o), _ptr(positions), _ptr(cos_cache),
                                          _ptr(sin_cache), T, H, D, 2 * half, P, G, _ptr(q),
                                          _ptr(s), _stream(o)))
    return q, s


def silu_f32_of_bf16(first_bits: int, n: int, device="cuda") -> torch.Tensor:
    """Diagnostic: the device silu of bf16 bit patterns first_bits .. + n - 1."""
    out = torch.empty((n,), dtype=torch.float32, device=device)
    L = load_library()
    _check("fp8_silu_f32_of_bf16",
           L.fp8_silu_f32_of_bf16(first_bits, n, _ptr(out), _stream(out)))
    return out


def requantize_weights(weights: Sequence[torch.Tensor], scale_fmt: int = SCALE_F32,
                       out: Sequence[Tuple[torch.Tensor, torch.Tensor]] = None
                       ) -> List[Tuple[torch.Tensor, torch.Tensor]]:
    """128x128-block quantization of every bf16 [N, K] weight in one batched
    call.  Returns [(E4M3 bytes [N, K], scales [N/128, K/128])] with fp32
    scales or uint8 E8M0 bytes.  ``out`` may supply preallocated outputs."""
    if len(weights) == 0:
        return []
    if scale_fmt not in (SCALE_F32, SCALE_E8M0):
        raise ValueError(f"scale_fmt must be SCALE_F32 or SCALE_E8M0, got {scale_fmt}")
    if out is not None and len(out) != len(weights):
        raise ValueError("out must hold one (q, s) pair per weight")
    _need(weights[0], torch.bfloat16, 2, "weights[0]")
    dev = weights[0].device
    sdt = torch.float32 if scale_fmt == SCALE_F32 else torch.uint8
    descs = (_WeightDesc * len(weights))()
    results = []
    for i, w in enumerate(weights):
        _need(w, torch.bfloat16, 2, f"weights[{i}]")
        if w.device != dev:
            raise ValueError(f"weights[{i}] must be on {dev}")
        N, K = w.shape
        q, s = _out_pair(None if out is None else out[i], (N, K), sdt, (N // 128, K // 128), dev)
        descs[i] = _WeightDesc(w.data_ptr(), q.data_ptr(), s.data_ptr(), N, K)
        results.append((q, s))
    _on_gpu(weights[0], "weights[0]")
    L = load_library()
    if L.fp8_requantize_workspace_size(len(weights)) != 0:
        raise RuntimeError("fp8_requantize_weights: the library asks for a workspace")
    _check("fp8_requantize_weights",
           L.fp8_requantize_weights(descs, len(weights), scale_fmt, None, 0, _stream(weights[0])))
    return results


def quantize_tensors(tensors: Sequence[torch.Tensor],
                     out: Sequence[Tuple[torch.Tensor, torch.Tensor]] = None
                     ) -> List[Tuple[torch.Tensor, torch.Tensor]]:
    """Per-tensor quantization of every contiguous bf16 tensor in one batched
    call (e.g. the K and V caches of every layer).  Returns [(E4M3 bytes of
    the tensor's shape, fp32 scale [1])]."""
    if len(tensors) == 0:
        return []
    if out is not None and len(out) != len(tensors):
        raise ValueError("out must hold one (q, s) pair per tensor")
    descs = (_TensorDesc * len(tensors))()
    results = []
    dev = None
    for i, x in enumerate(tensors):
        if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16:
            raise TypeError(f"tensors[{i}] must be a bf16 torch.Tensor")
        if not x.is_contiguous():
            raise ValueError(f"tensors[{i}] must be contiguous")
        dev = x.device if dev is None else dev
        if x.device != dev:
            raise ValueError(f"tensors[{i}] must be on {dev}")
        q, s = _out_pair(None if out is None else out[i], tuple(x.shape), torch.float32, (1,),
                         dev)
        descs[i] = _TensorDesc(x.data_ptr(), q.data_ptr(), s.data_ptr(), x.numel())
        results.append((q, s))
    _on_gpu(tensors[0], "tensors[0]")
    L = load_library()
    _check("fp8_quantize_tensors", L.fp8_quantize_tensors(descs, len(tensors), _stream(tensors[0])))
    return results


def quantize_tensor(x: torch.Tensor, out=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """One scale for the whole bf16 tensor: (E4M3 bytes, fp32 scale [1])."""
    return quantize_tensors([x], None if out is None else [out])[0]


# ----------------------------------------------------------------- GEMMs --
def _workspace(nbytes: int, workspace, device):
    """The GEMM's partial-tile workspace: ``workspace`` (a uint8 tensor of at
    least ``nbytes`` bytes on ``device``) when given, else a new one from
    torch's allocator (under graph capture, the graph's memory pool)."""
    if nbytes == 0:
        return None, 0
    if workspace is None:
        return torch.empty((nbytes,), dtype=torch.uint8, device=device), nbytes
    if not isinstance(workspace, torch.Tensor) or workspace.dtype != torch.uint8:
        raise TypeError("workspace must be a uint8 torch.Tensor")
    if not workspace.is_contiguous() or workspace.device != device:
        raise ValueError(f"workspace must be contiguous and on {device}")
    if workspace.numel() < nbytes:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {nbytes}")
    return workspace, workspace.numel()


def gemm_workspace_size(M: int, N: int, K: int, gran: int = GRAN_BLOCK) -> int:
    """Bytes of workspace gemm_a8w8_scaled uses for this shape (0: none)."""
    return int(load_library().fp8_gemm_workspace_size(M, N, K, gran))


def gemm_a8w8_scaled(a: Tuple[torch.Tensor, torch.Tensor], w: Tuple[torch.Tensor, torch.Tensor],
                     gran: int = GRAN_BLOCK, out: torch.Tensor = None,
                     workspace: torch.Tensor = None) -> torch.Tensor:
    """Y = X W^T in bf16 from (q, s) pairs: a = (E4M3 [M, K], scales),
    w = (E4M3 [N, K], scales).  BLOCK: scales [M, K/128] and [N/128, K/128];
    ROW: [M] and [N].  ``workspace`` may supply the partial-tile buffer
    (uint8, at least gemm_workspace_size bytes); by default one is taken from
    torch's allocator for the call."""
    if gran not in (GRAN_BLOCK, GRAN_ROW):
        raise ValueError(f"gran must be GRAN_BLOCK or GRAN_ROW, got {gran}")
    qa, sa = a
    qw, sw = w
    if not isinstance(qa, torch.Tensor) or qa.dim() != 2 or qa.dtype not in _CODES:
        raise TypeError("a[0] must be a 2-D uint8 / float8_e4m3fn tensor")
    if not isinstance(qw, torch.Tensor) or qw.dim() != 2 or qw.dtype not in _CODES:
        raise TypeError("w[0] must be a 2-D uint8 / float8_e4m3fn tensor")
    M, K = qa.shape
    N = qw.shape[0]
    dev = qa.device
    _need_buf(qa, _CODES, (M, K), "a[0]", dev)
    _need_buf(qw, _CODES, (N, K), "w[0]", dev)
    if gran == GRAN_BLOCK:
        _need_buf(sa, _F32, (M, K // 128), "a[1]", dev)
        _need_buf(sw, _F32, (N // 128, K // 128), "w[1]", dev)
    else:
        _need_buf(sa, _F32, (M,), "a[1]", dev)
        _need_buf(sw, _F32, (N,), "w[1]", dev)
    if out is not None:
        _need_buf(out, _BF16, (M, N), "out", dev)
    _on_gpu(qa, "a[0]")
    L = load_library()
    ws, ws_bytes = _workspace(int(L.fp8_gemm_workspace_size(M, N, K, gran)), workspace, dev)
    y = out if out is not None else torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    _check("fp8_gemm_a8w8_scaled",
           L.fp8_gemm_a8w8_scaled(_ptr(qa), _ptr(qw), _ptr(sa), _ptr(sw), None, _ptr(y), M, N, K,
                                  gran, _ptr(ws), ws_bytes, _stream(qa)))
    return y


def batched_gemm_mxscale_workspace_size(B: int, M: int, N: int, K: int) -> int:
    """Bytes of workspace batched_gemm_a8w8_mxscale uses for this shape."""
    return int(load_library().fp8_batched_gemm_mxscale_workspace_size(B, M, N, K))


def batched_gemm_a8w8_mxscale(a: Tuple[torch.Tensor, torch.Tensor],
                              w: Tuple[torch.Tensor, torch.Tensor],
                              out: torch.Tensor = None,
                              workspace: torch.Tensor = None) -> torch.Tensor:
    """E8M0-scaled GEMM.  Batched: a = (E4M3 [M, B, K], bytes [M, B, K/128]),
    w = (E4M3 [B, N, K], bytes [B, N/128, K/128]) -> bf16 [M, B, N].  Dense:
    a = ([M, K], [M, K/128]), w = ([N, K], [N/128, K/128]) -> [M, N].
    ``workspace`` as for gemm_a8w8_scaled."""
    qa, sa = a
    qw, sw = w
    if not isinstance(qa, torch.Tensor) or qa.dtype not in _CODES or qa.dim() not in (2, 3):
        raise TypeError("a[0] must be a 2-D or 3-D uint8 / float8_e4m3fn tensor")
    dense = qa.dim() == 2
    if dense:
        M, K = qa.shape
        B = 1
        N = qw.shape[0] if isinstance(qw, torch.Tensor) and qw.dim() == 2 else -1
        a_shape, sa_shape = (M, K), (M, K // 128)
        w_shape, sw_shape = (N, K), (N // 128, K // 128)
        shape = (M, N)
    else:
        M, B, K = qa.shape
        N = qw.shape[1] if isinstance(qw, torch.Tensor) and qw.dim() == 3 else -1
        a_shape, sa_shape = (M, B, K), (M, B, K // 128)
        w_shape, sw_shape = (B, N, K), (B, N // 128, K // 128)
        shape = (M, B, N)
    dev = qa.device
    if N < 0:
        raise ValueError(f"w[0] must have {qa.dim()} dims")
    _need_buf(qa, _CODES, a_shape, "a[0]", dev)
    _need_buf(qw, _CODES, w_shape, "w[0]", dev)
    _need_buf(sa, _U8, sa_shape, "a[1]", dev)
    _need_buf(sw, _U8, sw_shape, "w[1]", dev)
    if out is not None:
        _need_buf(out, _BF16, shape, "out", dev)
    _on_gpu(qa, "a[0]")
    L = load_library()
    ws, ws_bytes = _workspace(int(L.fp8_batched_gemm_mxscale_workspace_size(B, M, N, K)),
                              workspace, dev)
    y = out if out is not None else torch.empty(shape, dtype=torch.bfloat16, device=dev)
    _check("fp8_batched_gemm_a8w8_mxscale",
           L.fp8_batched_gemm_a8w8_mxscale(_ptr(qa), _ptr(qw), _ptr(sa), _ptr(sw), _ptr(y), B, M,
                                           N, K, _ptr(ws), ws_bytes, _stream(qa)))
    return y


def grouped_gemm_a8w8_scaled(a: Tuple[torch.Tensor, torch.Tensor],
                             w: Tuple[torch.Tensor, torch.Tensor], offsets: torch.Tensor,
                             out: torch.Tensor = None) -> torch.Tensor:
    """MoE grouped block-scaled GEMM: a = (E4M3 [T, K], [T, K/128]),
    w = (E4M3 [E, N, K], [E, N/128, K/128]), offsets int32 [E+1] on the device."""
    qa, sa = a
    qw, sw = w
    if not isinstance(qa, torch.Tensor) or qa.dim() != 2 or qa.dtype not in _CODES:
        raise TypeError("a[0] must be a 2-D uint8 / float8_e4m3fn tensor")
    if not isinstance(qw, torch.Tensor) or qw.dim() != 3 or qw.dtype not in _CODES:
        raise TypeError("w[0] must be a 3-D uint8 / float8_e4m3fn tensor")
    T, K = qa.shape
    E, N, _ = qw.shape
    dev = qa.device
    _need_buf(qa, _CODES, (T, K), "a[0]", dev)
    _need_buf(qw, _CODES, (E, N, K), "w[0]", dev)
    _need_buf(sa, _F32, (T, K // 128), "a[1]", dev)
    _need_buf(sw, _F32, (E, N // 128, K // 128), "w[1]", dev)
    _need_buf(offsets, (torch.int32,), (E + 1,), "offsets", dev)
    if out is not None:
        _need_buf(out, _BF16, (T, N), "out", dev)
    _on_gpu(qa, "a[0]")
    y = out if out is not None else torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    L = load_library()
    _check("fp8_grouped_gemm_a8w8_scaled",
           L.fp8_grouped_gemm_a8w8_scaled(_ptr(qa.view(torch.uint8)), _ptr(qw.view(torch.uint8)),
                                          _ptr(sa), _ptr(sw), _ptr(offsets), _ptr(y), T, E, N, K,
                                          _stream(qa)))
    return y


def bf16_round_f32_bits(first_bits: int, n: int, device="cuda") -> torch.Tensor:
    """Diagnostic: bf16 bit patterns (as int16) of the rounded fp32 bit
    patterns first_bits .. +n-1."""
    out = torch.empty((n,), dtype=torch.int16, device=device)
    L = load_library()
    _check("fp8_bf16_round_f32_bits",
           L.fp8_bf16_round_f32_bits(first_bits, n, _ptr(out), _stream(out)))
    return out


def encode_f32_bits(first_bits: int, n: int, device="cuda") -> torch.Tensor:
    """Diagnostic: E4M3 codes of the fp32 bit patterns first_bits .. +n-1."""
    q = torch.empty((n,), dtype=torch.uint8, device=device)
    L = load_library()
    _check("fp8_encode_f32_bits",
           L.fp8_encode_f32_bits(first_bits, n, _ptr(q), _stream(q)))
    return q
