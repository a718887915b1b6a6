"""GPU parity of the scaled GEMMs against the oracle's fp64 dequantize-then-
multiply: per output row, max |gpu - oracle| <= 1e-2 * max |oracle row|.

The GPU side quantizes and multiplies with the library; the oracle quantizes
the same bf16 inputs itself and multiplies in fp64.  Shapes: small ones that
span several 128 x 128 tiles with ragged M, the tiny linear, every dense
linear at M = 256 and M = 8192 (sampled rows), the per-row workload
(RMSNorm + per-token activations x per-row weights), and the MoE grouped GEMM
at full size (sampled rows, at least one per expert) plus small ragged cases
with empty experts.
"""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_amd as fp8
import oracle
import synth
from tests.gpu_util import (GEMM_ROW_TOL, assert_rows_close, dev, ensure_library, host,
                            sample_rows, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_library()


def _block_pipeline(X, W, rows=None):
    """GPU: quantize X (1x128) and W (128x128), GEMM.  Oracle: same from bf16."""
    qa, sa = fp8.quantize_block(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev()) if not W.is_cuda else W], fp8.SCALE_F32)
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    Xh = X if rows is None else X[torch.as_tensor(rows)]
    oqa, osa = oracle.quantize_block(Xh)
    oqw, osw = oracle.quantize_weight_block(W.cpu(), 0)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_BLOCK)
    return y, ref


def test_tiny_linear():
    say("block GEMM tiny 16x256x256")
    X, W = synth.tiny_linear(seed=0)
    y, ref = _block_pipeline(X, W)
    assert_rows_close(y, ref, what="tiny")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (16, 256, 256), (130, 384, 512),
                                   (300, 256, 1024), (257, 128, 4096), (64, 640, 384)])
def test_block_small_shapes(M, N, K):
    say(f"block GEMM {M}x{N}x{K}")
    X = synth.act_col_outliers(M, K, seed=M + N + K)
    W = synth.weight(N, K, seed=N + K)
    y, ref = _block_pipeline(X, W)
    assert_rows_close(y, ref, what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1024, 256, 256), (1100, 768, 640), (2047, 512, 1152),
                                   (8200, 2304, 256), (1024, 512, 128), (4352, 4096, 128),
                                   (700, 16384, 256)])
def test_block_large_m_shapes(M, N, K):
    # 8200 x 2304: 33 x 9 = 297 tiles of 256 x 256 on 256 workgroups, so some
    # workgroups run two tiles; the last row tile holds 8 rows.  K = 128: one
    # K block per tile (1024 x 512: one block per workgroup; 4352 x 4096: 272
    # tiles, a new tile at every block of the workgroups that run two).
    # 700 x 16384: 3 x 64 = 192 tiles, enough for the large-M kernel below
    # M = 1024; the last row tile holds 188 rows
    say(f"block GEMM (large-M kernel) {M}x{N}x{K}")
    X = synth.act_col_outliers(M, K, seed=M + N + K)
    W = synth.weight(N, K, seed=N + K + 1)
    y, ref = _block_pipeline(X, W)
    assert_rows_close(y, ref, what=f"{M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (130, 384, 512), (77, 256, 5120),
                                   (1100, 768, 640), (1024, 256, 4096), (8200, 2304, 256),
                                   (700, 16384, 256)])
def test_row_small_shapes(M, N, K):
    say(f"row GEMM {M}x{N}x{K}")
    X = synth.act_col_outliers(M, K, seed=M + 3)
    W = synth.weight(N, K, seed=K + 5)
    qa, sa = fp8.quantize_token(X.to(dev()))
    qw, sw = fp8.quantize_token(W.to(dev()))
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_ROW)
    oqa, osa = oracle.quantize_token(X)
    oqw, osw = oracle.quantize_token(W)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_ROW)
    assert_rows_close(y, ref, what=f"row {M}x{N}x{K}")


@pytest.mark.parametrize("name", list(synth.DENSE_SHAPES))
@pytest.mark.parametrize("M", synth.DENSE_M)
def test_dense_linears_full_size_sampled(name, M):
    N, K = synth.DENSE_SHAPES[name]
    say(f"block GEMM {name} M={M} ({M}x{N}x{K}), sampled rows")
    X, W = synth.dense_linear(name, M, seed=11)
    rows = sample_rows(M, 24, seed=M + N)
    y, ref = _block_pipeline(X, W, rows=rows)
    assert_rows_close(y, ref, rows=rows, what=f"{name} M={M}")


# Small-M shapes run stream-K: the tiles' K steps are split evenly over the
# workgroups and a tile cut between workgroups is summed, in a fixed order, by
# a second kernel.
@pytest.mark.parametrize("M,N,K", [(200, 8960, 640),    # 140 tiles, ranges of 2-3 steps
                                   (1000, 5120, 384),   # 320 tiles (> one per CU)
                                   (3, 1024, 12288),    # 8 tiles, 96 steps each
                                   (129, 128, 128)])    # 2 tiles, 1 step each
def test_block_stream_k_shapes(M, N, K):
    say(f"block GEMM stream-K {M}x{N}x{K}")
    X = synth.act_col_outliers(M, K, seed=M + 2 * N + K)
    W = synth.weight(N, K, seed=N + 2 * K)
    y, ref = _block_pipeline(X, W)
    assert_rows_close(y, ref, what=f"{M}x{N}x{K}")


# Above 128 rows, a small-M GEMM with at least 8 K steps per workgroup runs
# stream-K on 256 x 128 tiles: scales of 4 K blocks loaded together when
# K / 128 % 4 == 0, per step otherwise; ragged M over two row tiles.
DK_SHAPES = [(256, 8192, 4096),    # 64 tiles x 32 steps, grouped scale loads
             (300, 2048, 8192),    # 2 row tiles, the second 44 rows
             (160, 16384, 2176)]   # K / 128 = 17: per-step scale loads


@pytest.mark.parametrize("M,N,K", DK_SHAPES)
def test_block_stream_k_256_row_tiles(M, N, K):
    say(f"block GEMM stream-K 256-row tiles {M}x{N}x{K}, sampled rows")
    X = synth.act_col_outliers(M, K, seed=M + N + 3 * K)
    W = synth.weight(N, K, seed=N + 3 * K)
    rows = sample_rows(M, 24, seed=M + K)
    y, ref = _block_pipeline(X, W, rows=rows)
    assert_rows_close(y, ref, rows=rows, what=f"dk {M}x{N}x{K}")
    y2, _ = _block_pipeline(X, W, rows=[0])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # fixed-order reduce


@pytest.mark.parametrize("M,N,K", DK_SHAPES)
def test_row_stream_k_256_row_tiles(M, N, K):
    say(f"row GEMM stream-K 256-row tiles {M}x{N}x{K}, sampled rows")
    X = synth.act_col_outliers(M, K, seed=M + 5)
    W = synth.weight(N, K, seed=K + 7)
    qa, sa = fp8.quantize_token(X.to(dev()))
    qw, sw = fp8.quantize_token(W.to(dev()))
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_ROW)
    rows = sample_rows(M, 24, seed=M + N)
    oqa, osa = oracle.quantize_token(X[torch.as_tensor(rows)])
    oqw, osw = oracle.quantize_token(W)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_ROW)
    assert_rows_close(y, ref, rows=rows, what=f"row dk {M}x{N}x{K}")


# When whole tiles fill at least 3/4 of the CUs evenly, the small-M kernels
# deal out whole tiles (no split tiles, no reduce): 192 tiles of 256 x 128,
# 384 tiles of 128 x 128 (two per workgroup), 192 tiles of 128 x 128.
WHOLE_SHAPES = [(200, 24576, 2048), (256, 24576, 1024), (100, 24576, 1024)]


@pytest.mark.parametrize("gran", ["block", "row", "mx"])
@pytest.mark.parametrize("M,N,K", WHOLE_SHAPES)
def test_small_m_whole_tile_grids(M, N, K, gran):
    say(f"{gran} GEMM small-M whole-tile grid {M}x{N}x{K}, sampled rows")
    X = synth.act_col_outliers(M, K, seed=M + K + 17)
    W = synth.weight(N, K, seed=N + K + 19)
    rows = sample_rows(M, 16, seed=M + 3 * K)
    if gran == "block":
        y, ref = _block_pipeline(X, W, rows=rows)
    elif gran == "mx":
        y, ref = _mx_pipeline(X, W, rows=rows)
    else:
        qa, sa = fp8.quantize_token(X.to(dev()))
        qw, sw = fp8.quantize_token(W.to(dev()))
        y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_ROW)
        oqa, osa = oracle.quantize_token(X[torch.as_tensor(rows)])
        oqw, osw = oracle.quantize_token(W)
        ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_ROW)
    assert_rows_close(y, ref, rows=rows, what=f"{gran} whole {M}x{N}x{K}")


def test_stream_k_repeatable_across_interleaved_shapes():
    """Outputs do not depend on timing or on the shapes run before: A, B, A
    give bit-identical A outputs, all within tolerance of the oracle."""
    say("stream-K repeatability: shapes A, B, A on one stream")
    shapes = [(256, 4096, 12288), (96, 6144, 4096)]
    ops = []
    for i, (M, N, K) in enumerate(shapes):
        X = synth.act_col_outliers(M, K, seed=40 + i)
        W = synth.weight(N, K, seed=50 + i)
        qa, sa = fp8.quantize_block(X.to(dev()))
        (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
        ops.append(((qa, sa), (qw, sw), X, W))
    outs = []
    for idx in (0, 1, 0, 0):
        a, w, _, _ = ops[idx]
        outs.append(fp8.gemm_a8w8_scaled(a, w, fp8.GRAN_BLOCK))
    torch.cuda.synchronize()
    for o in outs[2:]:
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    for idx, o in ((0, outs[0]), (1, outs[1])):
        _, _, X, W = ops[idx]
        oqa, osa = oracle.quantize_block(X)
        oqw, osw = oracle.quantize_weight_block(W, 0)
        ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_BLOCK)
        assert_rows_close(o, ref, what=f"shape {shapes[idx]}")


def test_stream_k_concurrent_streams():
    """Small-M GEMMs issued on two streams at once (one on 256-row tiles, one
    on 128-row tiles): each stream has its own stream-K workspace, so the
    overlapping launches do not mix partials.  Every result matches the same
    GEMM run alone."""
    say("stream-K GEMMs on two concurrent streams")
    shapes = [(256, 4096, 12288), (200, 6144, 4096)]
    ops, solo = [], []
    for i, (M, N, K) in enumerate(shapes):
        X = synth.act_col_outliers(M, K, seed=80 + i)
        W = synth.weight(N, K, seed=90 + i)
        qa, sa = fp8.quantize_block(X.to(dev()))
        (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
        ops.append(((qa, sa), (qw, sw)))
        solo.append(fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[], []]
    for _ in range(6):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                outs[i].append(fp8.gemm_a8w8_scaled(ops[i][0], ops[i][1], fp8.GRAN_BLOCK))
    torch.cuda.synchronize()
    for i in range(2):
        for o in outs[i]:
            assert torch.equal(o.view(torch.int16), solo[i].view(torch.int16)), f"stream {i}"


def test_small_m_gemm_in_graph_capture():
    """Under graph capture no workspace is allocated for the capturing stream,
    so the small-M GEMM runs the plain persistent kernel; every replay (with
    eager work and synchronizations between them) matches the eager stream-K
    result within tolerance of the oracle."""
    say("small-M GEMM captured in a HIP graph, 3 replays")
    M, N, K = 256, 4096, 4096
    X = synth.act_col_outliers(M, K, seed=61)
    W = synth.weight(N, K, seed=62)
    qa, sa = fp8.quantize_block(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
    eager = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK, out=y)
    oqa, osa = oracle.quantize_block(X)
    oqw, osw = oracle.quantize_weight_block(W, 0)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_BLOCK)
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_rows_close(y, ref, what=f"replay {rep}")
        diff = (y.float() - eager.float()).abs().max().item()
        assert diff <= 1e-2 * eager.float().abs().max().item()
        _ = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)  # eager work between


def test_large_m_block_gemm_repeatable():
    # 48 tiles per workgroup with two K blocks each: a tile boundary every
    # other block, where the kernel stores a tile while the next blocks' loads
    # are in flight; three runs must give the same bits, and sampled rows
    # (incl. the ragged last tile) match the oracle
    M, N, K = 12288 + 100, 8192, 256
    say(f"block GEMM repeatable {M}x{N}x{K}")
    X = synth.act_col_outliers(M, K, seed=21)
    W = synth.weight(N, K, seed=22)
    qa, sa = fp8.quantize_block(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
    ys = [fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK) for _ in range(3)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    rows = np.unique(np.concatenate([sample_rows(M, 12, seed=3), np.arange(M - 100, M)]))
    y, ref = _block_pipeline(X, W, rows=rows)
    assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))
    assert_rows_close(y, ref, rows=rows, what="repeatable")


def test_ragged_m_full_k():
    M, N, K = 8192 + 37, 512, 12288
    say(f"block GEMM ragged {M}x{N}x{K}, sampled rows incl. the last tile")
    X = synth.act_col_outliers(M, K, seed=5)
    W = synth.weight(N, K, seed=6)
    rows = np.unique(np.concatenate([sample_rows(M, 16, seed=1), np.arange(M - 40, M)]))
    y, ref = _block_pipeline(X, W, rows=rows)
    assert_rows_close(y, ref, rows=rows, what="ragged")


def test_rms_row_workload_full_size_sampled():
    say("rmsnorm_quant -> row GEMM 4096x12288x5120, sampled rows")
    h, gamma = synth.rms_inputs(seed=0)
    W = synth.weight(synth.RMS_N, synth.RMS_K, seed=21)
    qa, sa = fp8.rmsnorm_quant(h.to(dev()), gamma.to(dev()), synth.RMS_EPS, 0)
    qw, sw = fp8.quantize_token(W.to(dev()))
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_ROW)
    rows = sample_rows(4096, 24, seed=3)
    oqa, osa = oracle.rmsnorm_quant(h[torch.as_tensor(rows)], gamma, synth.RMS_EPS)
    oqw, osw = oracle.quantize_token(W)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_ROW)
    assert_rows_close(y, ref, rows=rows, what="rms row")


def _grouped_pipeline(A, W, offsets, rows=None):
    E, N, K = W.shape
    qa, sa = fp8.quantize_block(A.to(dev()))
    Wd = W.to(dev()) if not W.is_cuda else W
    (qw, sw), = fp8.requantize_weights([Wd.reshape(E * N, K)], fp8.SCALE_F32)
    qw = qw.view(E, N, K)
    sw = sw.view(E, N // 128, K // 128)
    off = torch.as_tensor(offsets, dtype=torch.int32, device=dev())
    y = fp8.grouped_gemm_a8w8_scaled((qa, sa), (qw, sw), off)
    T = A.shape[0]
    if rows is None:
        rows = np.arange(T)
    rows = np.asarray(rows)
    oqa, osa = oracle.quantize_block(A[torch.as_tensor(rows)])
    expert_of = np.searchsorted(np.asarray(offsets), rows, side="right") - 1
    ref = np.zeros((rows.size, N))
    for e in np.unique(expert_of):
        sel = np.nonzero(expert_of == e)[0]
        oqw, osw = oracle.quantize_weight_block(W[int(e)].cpu(), 0)
        ref[sel] = oracle.gemm(oqa[sel], oqw, osa[sel], osw, oracle.GRAN_BLOCK)
    return y, ref, rows


def test_grouped_small_with_empty_experts():
    say("grouped GEMM small, empty experts")
    counts = [130, 0, 7, 0, 256, 1]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T, N, K = int(offsets[-1]), 256, 384
    A = synth.act_col_outliers(T, K, seed=8)
    W = synth.normal_bf16((len(counts), N, K), seed=9, std=0.02)
    y, ref, rows = _grouped_pipeline(A, W, offsets)
    assert_rows_close(y, ref, what="grouped small")


def test_grouped_rows_outside_offsets_untouched():
    say("grouped GEMM rows past offsets[E] untouched")
    offsets = np.array([0, 5, 5, 40], np.int32)
    T, N, K = 64, 128, 256
    A = synth.act_col_outliers(T, K, seed=1)
    W = synth.normal_bf16((3, N, K), seed=2, std=0.02)
    qa, sa = fp8.quantize_block(A.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.reshape(3 * N, K).to(dev())], fp8.SCALE_F32)
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device=dev())
    off = torch.as_tensor(offsets, device=dev())
    fp8.grouped_gemm_a8w8_scaled((qa, sa), (qw.view(3, N, K), sw.view(3, 1, 2)), off, out=y)
    assert torch.all(y[40:] == 7.0)
    assert not torch.all(y[:40] == 7.0)


def test_grouped_big_tiles_ragged_experts():
    """Experts averaging >= 192 rows take 256-row tiles: row counts around
    the tile size (0, 1, 255, 256, 257, ...) and a 128-column tail."""
    say("grouped GEMM, 256-row tiles, ragged experts, N % 256 == 128")
    counts = [0, 1, 255, 256, 257, 600, 900, 130]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T, N, K = int(offsets[-1]), 384, 384
    A = synth.act_col_outliers(T, K, seed=18)
    W = synth.normal_bf16((len(counts), N, K), seed=19, std=0.02)
    y, ref, rows = _grouped_pipeline(A, W, offsets)
    assert_rows_close(y, ref, what="grouped big tiles")


def test_grouped_big_tiles_rows_outside_offsets_untouched():
    say("grouped GEMM, 256-row tiles, rows outside [offsets[0], offsets[E]) untouched")
    offsets = np.array([10, 300, 300, 1700], np.int32)
    T, N, K = 2000, 256, 256
    A = synth.act_col_outliers(T, K, seed=21)
    W = synth.normal_bf16((3, N, K), seed=22, std=0.02)
    qa, sa = fp8.quantize_block(A.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.reshape(3 * N, K).to(dev())], fp8.SCALE_F32)
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device=dev())
    off = torch.as_tensor(offsets, device=dev())
    fp8.grouped_gemm_a8w8_scaled((qa, sa), (qw.view(3, N, K), sw.view(3, 2, 2)), off, out=y)
    assert torch.all(y[:10] == 7.0) and torch.all(y[1700:] == 7.0)
    oqa, osa = oracle.quantize_block(A)
    for e in (0, 2):
        a, b = int(offsets[e]), int(offsets[e + 1])
        oqw, osw = oracle.quantize_weight_block(W[e], 0)
        ref = oracle.gemm(oqa[a:b], oqw, osa[a:b], osw, oracle.GRAN_BLOCK)
        assert_rows_close(y[a:b], ref, what=f"expert {e}")


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_grouped_moe_full_size_sampled(which):
    say(f"grouped GEMM MoE {which} full size, sampled rows (>= 1 per expert)")
    A, W, offsets = synth.moe_inputs(which, seed=0)
    rng = np.random.default_rng(4)
    rows = []
    for e in range(len(offsets) - 1):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            rows += [a, b - 1, int(rng.integers(a, b))]
    rows = np.unique(np.array(rows))
    y, ref, rows = _grouped_pipeline(A, W, offsets, rows=rows)
    assert_rows_close(y, ref, rows=rows, what=f"moe {which}")


def test_moe_chain_gate_up_swiglu_down_sampled():
    """The MoE expert chain on the GPU: 1x128 quant of the routed rows ->
    grouped gate_up GEMM -> SwiGLU + 1x128 quant -> grouped down GEMM.  The
    oracle runs the same chain from the same bf16 inputs (its gate_up output
    rounded to bf16).  Tolerance: the sum of the two stages' bounds, 2e-2 of
    the row max.  Where the two sides' gate_up outputs differ by a bf16 ulp,
    a SwiGLU code can land one E4M3 step apart, so the second GEMM sees
    slightly different inputs on top of its own error."""
    say("MoE chain gate_up -> swiglu_quant -> down, full size, sampled rows")
    A, Wg, offsets = synth.moe_inputs("gate_up", seed=0)
    _, Wd, _ = synth.moe_inputs("down", seed=0)
    E, N1, K1 = Wg.shape
    _, N2, K2 = Wd.shape
    assert N1 == 2 * K2
    off = torch.as_tensor(offsets, dtype=torch.int32, device=dev())
    qa, sa = fp8.quantize_block(A.to(dev()))
    (qg, sg), (qd, sd) = fp8.requantize_weights(
        [Wg.to(dev()).reshape(E * N1, K1), Wd.to(dev()).reshape(E * N2, K2)], fp8.SCALE_F32)
    y1 = fp8.grouped_gemm_a8w8_scaled((qa, sa), (qg.view(E, N1, K1), sg.view(E, N1 // 128, -1)),
                                      off)
    q2, s2 = fp8.swiglu_quant(y1)
    y2 = fp8.grouped_gemm_a8w8_scaled((q2, s2), (qd.view(E, N2, K2), sd.view(E, N2 // 128, -1)),
                                      off)
    rng = np.random.default_rng(14)
    rows = []
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            rows += [a, int(rng.integers(a, b))]
    rows = np.unique(np.array(rows))
    oqa, osa = oracle.quantize_block(A[torch.as_tensor(rows)])
    expert_of = np.searchsorted(np.asarray(offsets), rows, side="right") - 1
    ref = np.zeros((rows.size, N2))
    for e in np.unique(expert_of):
        sel = np.nonzero(expert_of == e)[0]
        oqg, osg = oracle.quantize_weight_block(Wg[int(e)], 0)
        h = oracle.gemm(oqa[sel], oqg, osa[sel], osg, oracle.GRAN_BLOCK)
        hb = torch.from_numpy(h).float().to(torch.bfloat16)
        oq2, os2, _ = oracle.swiglu_quant(hb)
        oqd, osd = oracle.quantize_weight_block(Wd[int(e)], 0)
        ref[sel] = oracle.gemm(oq2, oqd, os2, osd, oracle.GRAN_BLOCK)
    assert_rows_close(y2, ref, rows=rows, what="moe chain", tol=2 * GEMM_ROW_TOL)


# --------------------------------------------------- E8M0 (MX) scaled GEMM --
def _mx_pipeline(X, W, rows=None):
    """GPU: 1x128 E8M0 activations, 128x128 E8M0 weights, MX GEMM.  Oracle:
    the same quantization from bf16, then the fp64 GEMM with the powers of
    two the bytes stand for."""
    qa, sa = fp8.quantize_block_e8m0(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev()) if not W.is_cuda else W], fp8.SCALE_E8M0)
    y = fp8.batched_gemm_a8w8_mxscale((qa, sa), (qw, sw))
    Xh = X if rows is None else X[torch.as_tensor(rows)]
    oqa, osa = oracle.quantize_block_e8m0(Xh)
    oqw, osw = oracle.quantize_weight_block(W.cpu(), 1)
    return y, oracle.mx_gemm(oqa, oqw, osa, osw)


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (16, 256, 256), (130, 384, 512),
                                   (1024, 256, 4096), (1100, 768, 640), (2047, 640, 1152),
                                   (8200, 2304, 256)])
def test_mx_dense_shapes(M, N, K):
    # N = 384, 640: the last 256-column tile holds 128 columns
    say(f"MX GEMM {M}x{N}x{K}")
    X = synth.act_col_outliers(M, K, seed=M + 2 * N + K)
    W = synth.weight(N, K, seed=N + 3 * K)
    y, ref = _mx_pipeline(X, W)
    assert_rows_close(y, ref, what=f"mx {M}x{N}x{K}")


def test_mx_batched_groups():
    M, B, N, K = 300, 3, 384, 512
    say(f"batched MX GEMM M={M} B={B} N={N} K={K}")
    X = synth.act_col_outliers(M * B, K, seed=91)          # rows (m, b) of [M, B, K]
    W = synth.normal_bf16((B * N, K), seed=92, std=0.02)   # [B, N, K] as [B*N, K]
    qa, sa = fp8.quantize_block_e8m0(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_E8M0)
    y = fp8.batched_gemm_a8w8_mxscale((qa.view(M, B, K), sa.view(M, B, K // 128)),
                                      (qw.view(B, N, K), sw.view(B, N // 128, K // 128)))
    oqa, osa = oracle.quantize_block_e8m0(X)
    oqw, osw = oracle.quantize_weight_block(W, 1)
    ref = oracle.batched_mx_gemm(oqa.reshape(M, B, K), oqw.reshape(B, N, K),
                                 osa.reshape(M, B, K // 128), osw.reshape(B, N // 128, K // 128))
    assert_rows_close(y.view(M * B, N), ref.reshape(M * B, N), what="batched mx")


def test_inverse_rope_quant_into_batched_mx_gemm():
    """The DeepSeek V4 output-projection path: inverse RoPE + E8M0 group quant
    of o [T, 64, 128] viewed as 8 groups of 1024, then the batched MX GEMM
    against per-group weights [8, 512, 1024].  The codes are bit-exact (the
    quantizer's own test), so the GEMM tolerance applies."""
    T, G, N = 512, synth.ROPE_GROUPS, 512
    say(f"inverse RoPE quant -> batched MX GEMM, T={T} groups={G} N={N}")
    o, pos = synth.rope_inputs(T, seed=44)
    cos, sin = synth.rope_cache()
    K = synth.ROPE_HEADS * synth.ROPE_HEAD_DIM // G
    W = synth.normal_bf16((G, N, K), seed=45, std=0.02)
    qa, sa = fp8.inverse_rope_group_quant(o.to(dev()), torch.as_tensor(pos, device=dev()),
                                          torch.as_tensor(cos, device=dev()),
                                          torch.as_tensor(sin, device=dev()), G)
    (qw, sw), = fp8.requantize_weights([W.to(dev()).reshape(G * N, K)], fp8.SCALE_E8M0)
    y = fp8.batched_gemm_a8w8_mxscale((qa, sa), (qw.view(G, N, K), sw.view(G, N // 128, -1)))
    rows = sample_rows(T, 48, seed=46)
    oq, os_, _ = oracle.inverse_rope_group_quant(o[torch.as_tensor(rows)], pos[rows], cos, sin,
                                                 synth.ROPE_DIM)
    oqw, osw = oracle.quantize_weight_block(W.reshape(G * N, K), 1)
    ref = oracle.batched_mx_gemm(oq.reshape(-1, G, K), oqw.reshape(G, N, K),
                                 os_.reshape(-1, G, K // 128), osw.reshape(G, N // 128, -1))
    got = y[torch.as_tensor(rows, device=dev())].reshape(rows.size * G, N)
    assert_rows_close(got, ref.reshape(rows.size * G, N), what="rope -> mx gemm")


@pytest.mark.parametrize("M,N,K", [(200, 8960, 640), (3, 1024, 12288), (256, 4096, 4096)])
def test_mx_small_m_stream_k(M, N, K):
    # dense small M takes the stream-K kernels with E8M0 scales: tiles split
    # across workgroups (200 x 8960: 140 tiles, ranges of 2-3 steps), a long K
    # over few tiles, and a decode-size linear
    say(f"MX GEMM small-M stream-K {M}x{N}x{K}")
    X = synth.act_col_outliers(M, K, seed=M + N + 7)
    W = synth.weight(N, K, seed=N + K + 9)
    y, ref = _mx_pipeline(X, W)
    assert_rows_close(y, ref, what=f"mx sk {M}x{N}x{K}")
    y2, _ = _mx_pipeline(X, W, rows=[0])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # fixed-order reduce


@pytest.mark.parametrize("M,N,K", DK_SHAPES)
def test_mx_stream_k_256_row_tiles(M, N, K):
    say(f"MX GEMM stream-K 256-row tiles {M}x{N}x{K}, sampled rows")
    X = synth.act_col_outliers(M, K, seed=M + N + 11)
    W = synth.weight(N, K, seed=N + K + 13)
    rows = sample_rows(M, 24, seed=M + 2 * K)
    y, ref = _mx_pipeline(X, W, rows=rows)
    assert_rows_close(y, ref, rows=rows, what=f"mx dk {M}x{N}x{K}")
    y2, _ = _mx_pipeline(X, W, rows=[0])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # fixed-order reduce


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_mx_dense_full_size_sampled(name):
    N, K = synth.DENSE_SHAPES[name]
    M = 8192
    say(f"MX GEMM {name} M={M} ({M}x{N}x{K}), sampled rows")
    X, W = synth.dense_linear(name, M, seed=13)
    rows = sample_rows(M, 24, seed=N + 5)
    y, ref = _mx_pipeline(X, W, rows=rows)
    assert_rows_close(y, ref, rows=rows, what=f"mx {name}")
