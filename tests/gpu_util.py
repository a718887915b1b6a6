"""Helpers for the GPU parity tests (GPU side via the C ABI, oracle on the CPU)."""
import os
import sys

import numpy as np
import torch

import fp8_w8a8_quantized_amd as fp8

# GEMM pass criterion: per output row, max |gpu - oracle| <= 1e-2 * max |oracle row|
GEMM_ROW_TOL = 1e-2


def ensure_library():
    if not os.path.exists(fp8.library_path()):
        from fp8_w8a8_quantized_amd import build

        build.build()
    fp8.load_library()


def dev():
    return torch.device("cuda:0")


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def say(msg: str) -> None:
    """Name the case on stdout before a GPU step (flushed)."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def assert_rows_close(y_gpu: torch.Tensor, ref: np.ndarray, rows=None, what="", tol=None):
    """y_gpu bf16 [R, N] (or the listed rows of it) vs fp64 oracle [R', N]:
    per row, max |gpu - oracle| <= tol * max |oracle row| (tol defaults to the
    one-GEMM bound)."""
    tol = GEMM_ROW_TOL if tol is None else tol
    y = y_gpu if rows is None else y_gpu[torch.as_tensor(rows, device=y_gpu.device)]
    got = host(y.float()).astype(np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    err = np.abs(got - ref).max(axis=1)
    rowmax = np.abs(ref).max(axis=1)
    bad = np.nonzero(err > tol * rowmax)[0]
    assert bad.size == 0, (f"{what}: {bad.size} rows out of tolerance, first {bad[:8]}, "
                           f"worst ratio {float((err / np.maximum(rowmax, 1e-300)).max()):.3e}")
    return float((err / np.maximum(rowmax, 1e-300)).max())


def sample_rows(M: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and n random distinct rows of [0, M), sorted."""
    rng = np.random.default_rng(seed)
    pick = set([0, M - 1]) | set(rng.choice(M, size=min(n, M), replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)


def assert_gemm_all_rows(y_gpu: torch.Tensor, oqa, osa, oqw, osw, gran, what="", tol=None,
                         chunk: int = 1024):
    """Every row of y_gpu [M, N] against the oracle's fp64 product of the
    quantized operands (codes and scales from the oracle's own quantizers):
    the weight is dequantized once (oracle.dequant_weight) and the rows are
    compared in chunks of ``chunk`` (oracle.dequant_act, then the fp64
    product, as oracle.gemm computes it)."""
    import oracle

    W = oracle.dequant_weight(oqw, osw, gran)
    M = y_gpu.shape[0]
    worst = 0.0
    for r0 in range(0, M, chunk):
        r1 = min(M, r0 + chunk)
        ref = oracle.dequant_act(oqa[r0:r1], osa[r0:r1], gran) @ W.T
        worst = max(worst, assert_rows_close(y_gpu[r0:r1], ref, what=f"{what} rows {r0}..{r1}",
                                             tol=tol))
    return worst


def bf16_from_f64(h: np.ndarray) -> torch.Tensor:
    """The nearest bf16 (ties to even) to each fp64 value, as a bf16 CPU
    tensor.  Rounding to fp32 first can land exactly on a bf16 midpoint the
    fp64 value is not on; such fp32 values are moved one fp32 ulp toward the
    fp64 value before the fp32 -> bf16 rounding, which then picks the side the
    fp64 value lies on."""
    import oracle

    f = h.astype(np.float32)
    bits = f.view(np.uint32)
    fix = ((bits & 0xFFFF) == 0x8000) & (f.astype(np.float64) != h)
    if np.any(fix):
        toward = np.where(h[fix] > f[fix], np.float32(np.inf), np.float32(-np.inf))
        f[fix] = np.nextafter(f[fix], toward)
    b = oracle.bf16_rne_array(f.reshape(-1)).reshape(h.shape)
    return torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
