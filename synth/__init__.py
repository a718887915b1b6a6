"""Seeded synthetic inputs shared by the oracle-side and the HIP-side of tests and
the benchmark.

This module holds random draws, bf16 rounding of those draws and MoE routing
(which rows go to which expert).  It holds none of the quantization or GEMM
arithmetic: scales, codes and products are computed only by the oracle and by
the HIP library, each on its own.

Two generators exist for every tensor:
  * host: numpy PCG64 (``np.random.default_rng(seed)``) fp32 draws, rounded to
    bf16 (round-to-nearest-even, by torch's dtype conversion);
  * device: torch's seeded Philox generator on a GPU, for tensors too large to
    draw on the host in reasonable time (the 36-layer policy).  A test that
    needs oracle values for such a tensor copies the sampled part to the host.

Workload recipes (sizes and distributions of the pages' configurations):
  tiny linear:    X [16, 256] ~ N(0, 1) with each entry x20 with prob. 0.01;
                  W [256, 256] ~ N(0, 0.02).
  dense linears:  X [M, K] ~ N(0, 1) with round(0.001 K) distinct whole
                  columns x50; W [N, K] ~ N(0, 0.02);
                  (N, K) in qkv (6144, 4096), o (4096, 4096),
                  gate_up (24576, 4096), down (4096, 12288); M in {256, 8192}.
  policy requant: 36 layers x the four weights above ~ N(0, 0.02).
  rmsnorm:        h = bf16(z * g_k), z ~ N(0, 1) [4096, 5120], g_k = exp(N(0, 1))
                  per column; gamma ~ U(0.5, 1.5) in bf16; eps = 1e-6;
                  W [12288, 5120] ~ N(0, 0.02).
  MoE:            logits [4096, 128] ~ N(0, 1); each token's top-8 experts by
                  logit (ties to the lower expert id); rows sorted by
                  (expert, token); X [4096, 2048] ~ N(0, 1) gathered to
                  [32768, 2048]; down-projection input [32768, 768] ~ N(0, 1);
                  W gate_up [128, 1536, 2048], down [128, 2048, 768] ~ N(0, 0.02).
  inverse RoPE:   o [T, 64 heads, 128] ~ N(0, 1) bf16 with the rotary part in
                  the last 64 dims of each head; positions = token index within
                  sequences of 2048; cos/sin fp32 [8192, 32] of angle
                  p * 10000^(-2i/64), computed in fp64 and rounded once
                  8192 tokens; the projection's weights [8 groups, 1024, 1024]
                  ~ N(0, 0.02) (shapes are synthetic: the pages give none).
  KV cache:       per layer K and V [8192 tokens, 8 KV heads x 128] (the
                  Qwen3-8B-shaped attention of the dense linears); K ~ N(0, 1)
                  with one whole column x50 (an outlier channel), V ~ N(0, 1);
                  36 layers, one per-tensor scale each for K and V.
"""
from __future__ import annotations

import numpy as np
import torch

DENSE_SHAPES = {  # name -> (N, K) of a Qwen3-8B-shaped linear, W is [N, K]
    "qkv": (6144, 4096),
    "o": (4096, 4096),
    "gate_up": (24576, 4096),
    "down": (4096, 12288),
}
DENSE_M = (256, 8192)
POLICY_LAYERS = 36

RMS_M, RMS_K, RMS_N, RMS_EPS = 4096, 5120, 12288, 1e-6

MOE_TOKENS, MOE_EXPERTS, MOE_TOPK = 4096, 128, 8
MOE_HIDDEN, MOE_INTER = 2048, 768

KV_TOKENS, KV_HEADS, KV_HEAD_DIM = 8192, 8, 128

ROPE_HEADS, ROPE_HEAD_DIM, ROPE_DIM, ROPE_GROUPS, ROPE_MAX_POS, ROPE_SEQ = 64, 128, 64, 8, 8192, 2048
ROPE_TOKENS, ROPE_OUT = 8192, 1024  # tokens per step; per-group output width of the projection


def _is_dev(device) -> bool:
    return torch.device(device).type != "cpu"


def to_bf16(a: np.ndarray) -> torch.Tensor:
    """fp32 numpy array -> bf16 CPU tensor (round to nearest even)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (host copy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def normal_f32(shape, seed: int, std: float = 1.0, device="cpu"):
    if _is_dev(device):
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(std)


def normal_bf16(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    a = normal_f32(shape, seed, std, device)
    if isinstance(a, torch.Tensor):
        return a.to(torch.bfloat16)
    return to_bf16(a)


def weight(N: int, K: int, seed: int, device="cpu") -> torch.Tensor:
    return normal_bf16((N, K), seed, 0.02, device)


def act_entry_outliers(M: int, K: int, seed: int, p: float = 0.01, mult: float = 20.0):
    """N(0, 1) with each entry independently multiplied by ``mult`` w.p. ``p``."""
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((M, K), dtype=np.float32)
    hit = rng.random((M, K)) < p
    z[hit] *= np.float32(mult)
    return to_bf16(z)


def act_col_outliers(M: int, K: int, seed: int, frac: float = 0.001, mult: float = 50.0,
                     device="cpu"):
    """N(0, 1) with round(frac * K) distinct whole columns multiplied by ``mult``."""
    ncols = int(round(frac * K))
    rng = np.random.default_rng(seed + 7919)
    cols = np.sort(rng.choice(K, size=ncols, replace=False)) if ncols else np.zeros(0, int)
    z = normal_f32((M, K), seed, 1.0, device)
    if isinstance(z, torch.Tensor):
        if ncols:
            z[:, torch.as_tensor(cols, device=z.device)] *= mult
        return z.to(torch.bfloat16)
    if ncols:
        z[:, cols] *= np.float32(mult)
    return to_bf16(z)


def tiny_linear(seed: int = 0):
    """Tiny blockwise linear: X [16, 256], W [256, 256]."""
    X = act_entry_outliers(16, 256, seed)
    W = weight(256, 256, seed + 1)
    return X, W


def dense_linear(name: str, M: int, seed: int = 0, device="cpu"):
    N, K = DENSE_SHAPES[name]
    X = act_col_outliers(M, K, seed, device=device)
    W = weight(N, K, seed + 1, device=device)
    return X, W


def rms_inputs(M: int = RMS_M, K: int = RMS_K, seed: int = 0, device="cpu"):
    """h = bf16(z * g) with per-column lognormal gain; gamma ~ U(0.5, 1.5)."""
    rng = np.random.default_rng(seed + 104729)
    g = np.exp(rng.standard_normal(K, dtype=np.float32)).astype(np.float32)
    gamma = to_bf16(rng.uniform(0.5, 1.5, size=K).astype(np.float32))
    z = normal_f32((M, K), seed, 1.0, device)
    if isinstance(z, torch.Tensor):
        h = (z * torch.as_tensor(g, device=z.device)).to(torch.bfloat16)
        return h, gamma.to(z.device)
    return to_bf16(z * g[None, :]), gamma


def moe_routing(tokens: int = MOE_TOKENS, experts: int = MOE_EXPERTS, topk: int = MOE_TOPK,
                seed: int = 0):
    """Top-k experts per token by logit (softmax is monotone, so the set is the
    same); ties go to the lower expert id.  Rows are sorted by (expert, token).

    Returns (token_of_row [tokens*topk] int64, offsets [experts+1] int32)."""
    rng = np.random.default_rng(seed + 15485863)
    logits = rng.standard_normal((tokens, experts), dtype=np.float32)
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    tok = np.repeat(np.arange(tokens), topk)
    exp = order.reshape(-1)
    idx = np.lexsort((tok, exp))  # primary key expert, then token
    token_of_row = tok[idx].astype(np.int64)
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return token_of_row, offsets


def moe_inputs(which: str = "gate_up", seed: int = 0, tokens: int = MOE_TOKENS,
               experts: int = MOE_EXPERTS, device="cpu"):
    """MoE grouped GEMM inputs.  ``which`` = "gate_up" (N=1536, K=2048, rows are
    the routed tokens' hidden states) or "down" (N=2048, K=768, rows are
    independent N(0, 1) draws).  Returns (A_rows bf16 [T, K], W bf16 [E, N, K],
    offsets int32 [E+1])."""
    token_of_row, offsets = moe_routing(tokens, experts, MOE_TOPK, seed)
    T = token_of_row.size
    if which == "gate_up":
        N, K = 2 * MOE_INTER, MOE_HIDDEN
        X = normal_bf16((tokens, K), seed + 11, 1.0, device)
        A = X[torch.as_tensor(token_of_row, device=X.device)]
    else:
        N, K = MOE_HIDDEN, MOE_INTER
        A = normal_bf16((T, K), seed + 13, 1.0, device)
    W = normal_bf16((experts, N, K), seed + 17, 0.02, device)
    return A, W, offsets


def kv_cache(layer: int, seed: int = 0, tokens: int = KV_TOKENS, device="cpu"):
    """K and V of one layer, [tokens, KV_HEADS * KV_HEAD_DIM] bf16 each."""
    width = KV_HEADS * KV_HEAD_DIM
    k = act_col_outliers(tokens, width, seed + 2 * layer, device=device)
    v = normal_bf16((tokens, width), seed + 2 * layer + 1, 1.0, device)
    return k, v


def rope_cache(max_pos: int = ROPE_MAX_POS, rope_dim: int = ROPE_DIM, base: float = 10000.0):
    """cos and sin fp32 [max_pos, rope_dim / 2] of angle p * base^(-2i/rope_dim)."""
    inv = base ** (-np.arange(0, rope_dim, 2, dtype=np.float64) / rope_dim)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope_inputs(tokens: int, seed: int = 0, heads: int = ROPE_HEADS, head_dim: int = ROPE_HEAD_DIM,
                seq: int = ROPE_SEQ, device="cpu"):
    """o bf16 [tokens, heads, head_dim] ~ N(0, 1) and int64 positions (token
    index within consecutive sequences of `seq`)."""
    o = normal_bf16((tokens, heads, head_dim), seed, 1.0, device)
    pos = np.arange(tokens, dtype=np.int64) % seq
    return o, pos
