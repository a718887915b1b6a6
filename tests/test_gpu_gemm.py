"""GPU parity of the scaled GEMMs against the oracle's fp64 dequantize-then-
multiply: per output row, max |gpu - oracle| <= 1e-2 * max |oracle row|.

The GPU side quantizes and multiplies with the library; the oracle quantizes
the same bf16 inputs itself and multiplies in fp64.  Shapes: small ones that
span several 128 x 128 tiles with ragged M, the tiny linear, every dense
linear at M = 256 and M = 8192, the per-row workload (RMSNorm + per-token
activations x per-row weights), the MX-scaled linears at M = 8192, and the MoE
grouped GEMMs at full size plus small ragged cases with empty experts, seeded
sweeps of shapes and routings, and a chain of launches captured in a HIP graph.
Every test compares every output row (full-size outputs in chunks of rows).
"""
import numpy as np
import pytest
import torch

import fp8_w8a8_quantized_amd as fp8
import oracle
import synth
from tests.gpu_util import (GEMM_ROW_TOL, assert_gemm_all_rows, assert_rows_close,
                            bf16_from_f64, dev, ensure_library, host, say)

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


def _block_check(X, W, what):
    """GPU pipeline as _block_pipeline; every output row against the oracle."""
    qa, sa = fp8.quantize_block(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev()) if not W.is_cuda else W], fp8.SCALE_F32)
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    oqa, osa = oracle.quantize_block(X.cpu())
    oqw, osw = oracle.quantize_weight_block(W.cpu(), 0)
    assert_gemm_all_rows(y, oqa, osa, oqw, osw, oracle.GRAN_BLOCK, what=what)
    return y


def _row_check(X, W, what):
    """Per-token activations x per-row weights; every output row."""
    qa, sa = fp8.quantize_token(X.to(dev()))
    qw, sw = fp8.quantize_token(W.to(dev()))
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_ROW)
    oqa, osa = oracle.quantize_token(X.cpu())
    oqw, osw = oracle.quantize_token(W.cpu())
    assert_gemm_all_rows(y, oqa, osa, oqw, osw, oracle.GRAN_ROW, what=what)
    return y


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
def test_dense_linears_full_size(name, M):
    N, K = synth.DENSE_SHAPES[name]
    say(f"block GEMM {name} M={M} ({M}x{N}x{K}), every row")
    X, W = synth.dense_linear(name, M, seed=11)
    _block_check(X, W, f"{name} M={M}")


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
    say(f"block GEMM stream-K 256-row tiles {M}x{N}x{K}, every row")
    X = synth.act_col_outliers(M, K, seed=M + N + 3 * K)
    W = synth.weight(N, K, seed=N + 3 * K)
    y = _block_check(X, W, f"dk {M}x{N}x{K}")
    y2, _ = _block_pipeline(X, W, rows=[0])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # fixed-order reduce


@pytest.mark.parametrize("M,N,K", DK_SHAPES)
def test_row_stream_k_256_row_tiles(M, N, K):
    say(f"row GEMM stream-K 256-row tiles {M}x{N}x{K}, every row")
    X = synth.act_col_outliers(M, K, seed=M + 5)
    W = synth.weight(N, K, seed=K + 7)
    _row_check(X, W, f"row dk {M}x{N}x{K}")


# When whole tiles fill at least 3/4 of the CUs evenly, the small-M kernels
# deal out whole tiles (no split tiles, no reduce): 192 tiles of 256 x 128,
# 384 tiles of 128 x 128 (two per workgroup), 192 tiles of 128 x 128.
WHOLE_SHAPES = [(200, 24576, 2048), (256, 24576, 1024), (100, 24576, 1024)]


@pytest.mark.parametrize("gran", ["block", "row", "mx"])
@pytest.mark.parametrize("M,N,K", WHOLE_SHAPES)
def test_small_m_whole_tile_grids(M, N, K, gran):
    say(f"{gran} GEMM small-M whole-tile grid {M}x{N}x{K}, every row")
    X = synth.act_col_outliers(M, K, seed=M + K + 17)
    W = synth.weight(N, K, seed=N + K + 19)
    if gran == "block":
        _block_check(X, W, f"block whole {M}x{N}x{K}")
    elif gran == "mx":
        _mx_check(X, W, f"mx whole {M}x{N}x{K}")
    else:
        _row_check(X, W, f"row whole {M}x{N}x{K}")


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
    on 128-row tiles): each call takes its partial-tile workspace from torch's
    allocator on its own stream, so the overlapping launches do not mix
    partials.  Every result matches the same GEMM run alone."""
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


def _captured(fn, y):
    """Capture fn(y) in a HIP graph and return the graph."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn(y)
    return g


@pytest.mark.parametrize("M,N,K", [(256, 4096, 4096),     # 128-row stream-K, split tiles
                                   (256, 4096, 12288),    # 256-row stream-K, split tiles
                                   (256, 24576, 1024)])   # whole 256 x 128 tiles
def test_small_m_gemm_in_graph_capture(M, N, K):
    """Under graph capture the wrapper takes the workspace from the graph's
    memory pool, so the captured small-M GEMM runs the same kernels as eager
    (stream-K with its reduce, or whole tiles): every replay, with eager work
    and synchronizations between them, is bitwise equal to the eager result,
    which is within tolerance of the oracle."""
    say(f"small-M GEMM {M}x{N}x{K} captured in a HIP graph, 3 replays")
    X = synth.act_col_outliers(M, K, seed=61)
    W = synth.weight(N, K, seed=62)
    qa, sa = fp8.quantize_block(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
    eager = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    g = _captured(lambda out: fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK, out=out), y)
    oqa, osa = oracle.quantize_block(X)
    oqw, osw = oracle.quantize_weight_block(W, 0)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_BLOCK)
    assert_rows_close(eager, ref, what="eager")
    for rep in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        _ = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)  # eager work between


@pytest.mark.parametrize("M,N,K", [(256, 4096, 4096), (256, 4096, 12288), (3, 1024, 12288)])
def test_small_m_gemm_caller_workspace_and_none(M, N, K):
    """The caller's workspace: one buffer of the queried size reused across
    calls gives the bytes of the wrapper's own; a NULL workspace through the
    C ABI runs the plan without split tiles, within tolerance of the oracle."""
    import ctypes
    say(f"small-M GEMM {M}x{N}x{K}: caller workspace, then none")
    X = synth.act_col_outliers(M, K, seed=71)
    W = synth.weight(N, K, seed=72)
    qa, sa = fp8.quantize_block(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
    need = fp8.gemm_workspace_size(M, N, K, fp8.GRAN_BLOCK)
    assert need > 0
    ws = torch.empty((need,), dtype=torch.uint8, device=dev())
    base = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK)
    for _ in range(2):
        y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_BLOCK, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), base.view(torch.int16))
    L = fp8.load_library()
    y0 = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.fp8_gemm_a8w8_scaled(ctypes.c_void_p(qa.data_ptr()), ctypes.c_void_p(qw.data_ptr()),
                                ctypes.c_void_p(sa.data_ptr()), ctypes.c_void_p(sw.data_ptr()),
                                None, ctypes.c_void_p(y0.data_ptr()), M, N, K, fp8.GRAN_BLOCK,
                                None, 0, st)
    assert rc == 0
    oqa, osa = oracle.quantize_block(X)
    oqw, osw = oracle.quantize_weight_block(W, 0)
    ref = oracle.gemm(oqa, oqw, osa, osw, oracle.GRAN_BLOCK)
    assert_rows_close(y0, ref, what="no workspace")
    assert_rows_close(base, ref, what="workspace")


def test_large_m_block_gemm_repeatable():
    # 48 tiles per workgroup with two K blocks each: a tile boundary every
    # other block, where the kernel stores a tile while the next blocks' loads
    # are in flight; three runs must give the same bits, and sampled rows
    # (incl. the ragged last tile) match the oracle: every row
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
    y = _block_check(X, W, "repeatable")
    assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))


def test_ragged_m_full_k():
    M, N, K = 8192 + 37, 512, 12288
    say(f"block GEMM ragged {M}x{N}x{K}, every row")
    X = synth.act_col_outliers(M, K, seed=5)
    W = synth.weight(N, K, seed=6)
    _block_check(X, W, "ragged")


def test_rms_row_workload_full_size():
    say("rmsnorm_quant -> row GEMM 4096x12288x5120, every row")
    h, gamma = synth.rms_inputs(seed=0)
    W = synth.weight(synth.RMS_N, synth.RMS_K, seed=21)
    qa, sa = fp8.rmsnorm_quant(h.to(dev()), gamma.to(dev()), synth.RMS_EPS, 0)
    qw, sw = fp8.quantize_token(W.to(dev()))
    y = fp8.gemm_a8w8_scaled((qa, sa), (qw, sw), fp8.GRAN_ROW)
    oqa, osa = oracle.rmsnorm_quant(h, gamma, synth.RMS_EPS)
    oqw, osw = oracle.quantize_token(W)
    assert_gemm_all_rows(y, oqa, osa, oqw, osw, oracle.GRAN_ROW, what="rms row")


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


def test_grouped_big_tiles_ragged_full_columns():
    """Experts averaging >= 192 rows with N % 256 == 0 (the ping-pong
    kernel): counts on both sides of the 128- and 256-row boundaries of an
    expert's last tile (256 + 1, 256 + 128, 256 + 129, 512 + 1, ...)."""
    say("grouped GEMM, 256-row tiles, ragged experts, N % 256 == 0")
    counts = [0, 1, 255, 256, 257, 300, 384, 385, 600, 900, 130, 513, 640, 641]
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T, N, K = int(offsets[-1]), 512, 384
    A = synth.act_col_outliers(T, K, seed=23)
    W = synth.normal_bf16((len(counts), N, K), seed=24, std=0.02)
    y, ref, rows = _grouped_pipeline(A, W, offsets)
    assert_rows_close(y, ref, what="grouped ragged full columns")


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
def test_grouped_moe_full_size(which):
    say(f"grouped GEMM MoE {which} full size, every row")
    A, W, offsets = synth.moe_inputs(which, seed=0)
    y, ref, rows = _grouped_pipeline(A, W, offsets)
    assert rows.size == A.shape[0]
    assert_rows_close(y, ref, what=f"moe {which}")


def _moe_chain_oracle():
    """The expert chain on the oracle side, every row: 1x128 quant of the
    routed rows, per-expert fp64 gate_up, rounded to bf16 (nearest, from the
    fp64 value), SwiGLU + 1x128 quant, per-expert fp64 down."""
    A, Wg, offsets = synth.moe_inputs("gate_up", seed=0)
    _, Wd, _ = synth.moe_inputs("down", seed=0)
    E, N1, K1 = Wg.shape
    _, N2, K2 = Wd.shape
    assert N1 == 2 * K2
    oqa, osa = oracle.quantize_block(A)
    og = [oracle.quantize_weight_block(Wg[e], 0) for e in range(E)]
    od = [oracle.quantize_weight_block(Wd[e], 0) for e in range(E)]
    h = np.zeros((A.shape[0], N1))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            h[a:b] = oracle.gemm(oqa[a:b], og[e][0], osa[a:b], og[e][1], oracle.GRAN_BLOCK)
    hb = bf16_from_f64(h)
    oq2, os2, _ = oracle.swiglu_quant(hb)
    y2 = np.zeros((A.shape[0], N2))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y2[a:b] = oracle.gemm(oq2[a:b], od[e][0], os2[a:b], od[e][1], oracle.GRAN_BLOCK)
    return dict(A=A, Wg=Wg, Wd=Wd, offsets=offsets, h=h, hb=hb, q2=oq2, s2=os2, y2=y2, od=od)


@pytest.fixture(scope="module")
def moe_chain():
    return _moe_chain_oracle()


def _moe_weights_gpu(o):
    E, N1, K1 = o["Wg"].shape
    _, N2, K2 = o["Wd"].shape
    (qg, sg), (qd, sd) = fp8.requantize_weights(
        [o["Wg"].to(dev()).reshape(E * N1, K1), o["Wd"].to(dev()).reshape(E * N2, K2)],
        fp8.SCALE_F32)
    return ((qg.view(E, N1, K1), sg.view(E, N1 // 128, -1)),
            (qd.view(E, N2, K2), sd.view(E, N2 // 128, -1)))


def test_moe_chain_stagewise_full_size(moe_chain):
    """Each GPU stage of the MoE expert chain fed the oracle's output of the
    stage before, every row: gate_up within the GEMM bar; SwiGLU + 1x128
    quant of the oracle's bf16 gate_up output bit-exact; down on the oracle's
    SwiGLU codes within the GEMM bar."""
    say("MoE chain stage by stage on oracle-fed inputs, full size, every row")
    o = moe_chain
    off = torch.as_tensor(o["offsets"], dtype=torch.int32, device=dev())
    wg, wd = _moe_weights_gpu(o)
    qa, sa = fp8.quantize_block(o["A"].to(dev()))
    y1 = fp8.grouped_gemm_a8w8_scaled((qa, sa), wg, off)
    assert_rows_close(y1, o["h"], what="gate_up")
    q2, s2 = fp8.swiglu_quant(o["hb"].to(dev()))
    gq, gs = host(q2), host(s2)
    assert np.array_equal(gq, o["q2"]), f"SwiGLU codes differ at {np.argwhere(gq != o['q2'])[:5]}"
    assert np.array_equal(gs.view(np.uint32), o["s2"].view(np.uint32)), "SwiGLU scales differ"
    y2 = fp8.grouped_gemm_a8w8_scaled((torch.as_tensor(o["q2"], device=dev()),
                                       torch.as_tensor(o["s2"], device=dev())), wd, off)
    assert_rows_close(y2, o["y2"], what="down")


def test_moe_chain_end_to_end_full_size(moe_chain):
    """The whole chain on the GPU (1x128 quant -> grouped gate_up -> SwiGLU +
    quant -> grouped down) against the oracle's chain, every row.  The two
    sides' gate_up outputs may differ in their bf16 rounding (fp32 against
    fp64 sums), and where they do, SwiGLU codes of the down GEMM's input can
    differ too.  With d the difference of the two sides' dequantized down
    inputs and Q = |d| |W_down|^T, exact linear algebra bounds each row:
    |gpu - oracle| <= Q + 1e-2 (max|oracle row| + max Q), the down GEMM's own
    bar on its actual input plus the exact propagation of the input
    difference.  Rows whose inputs agree (Q = 0) are held to the plain GEMM
    bar; input codes may differ only in rows whose gate_up outputs differ."""
    say("MoE chain end to end on the GPU, full size, every row")
    o = moe_chain
    off = torch.as_tensor(o["offsets"], dtype=torch.int32, device=dev())
    wg, wd = _moe_weights_gpu(o)
    qa, sa = fp8.quantize_block(o["A"].to(dev()))
    y1 = fp8.grouped_gemm_a8w8_scaled((qa, sa), wg, off)
    q2, s2 = fp8.swiglu_quant(y1)
    y2 = fp8.grouped_gemm_a8w8_scaled((q2, s2), wd, off)
    g1 = host(y1.view(torch.int16)).view(np.uint16)
    gq, gs = host(q2), host(s2)
    h_same = np.all(g1 == synth.bf16_bits(o["hb"]), axis=1)
    d = (oracle.dequant_act(gq, gs, oracle.GRAN_BLOCK)
         - oracle.dequant_act(o["q2"], o["s2"], oracle.GRAN_BLOCK))
    d_rows = np.nonzero(np.any(d != 0, axis=1))[0]
    assert np.all(~h_same[d_rows]), "SwiGLU input codes differ in a row whose gate_up agrees"
    Q = np.zeros(o["y2"].shape)
    expert_of = np.searchsorted(np.asarray(o["offsets"]), d_rows, side="right") - 1
    for e in np.unique(expert_of):
        rows = d_rows[expert_of == e]
        Wde = np.abs(oracle.dequant_weight(*o["od"][int(e)], oracle.GRAN_BLOCK))
        Q[rows] = np.abs(d[rows]) @ Wde.T
    got = host(y2.float()).astype(np.float64)
    err = np.abs(got - o["y2"])
    rowmax = np.abs(o["y2"]).max(axis=1)
    bound = Q + GEMM_ROW_TOL * (rowmax + Q.max(axis=1))[:, None]
    bad = np.nonzero(np.any(err > bound, axis=1))[0]
    assert bad.size == 0, (f"{bad.size} rows out of bound, first {bad[:8]}; rows with differing "
                           f"down inputs: {d_rows.size}")
    same = np.setdiff1d(np.arange(got.shape[0]), d_rows)
    assert np.all(err[same].max(axis=1) <= GEMM_ROW_TOL * rowmax[same])
    print(f"rows with differing gate_up bf16: {int((~h_same).sum())}, with differing down "
          f"inputs: {d_rows.size}")


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


def _mx_check(X, W, what):
    """GPU pipeline as _mx_pipeline; every output row against the oracle (the
    E8M0 bytes read as the powers of two they stand for)."""
    qa, sa = fp8.quantize_block_e8m0(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev()) if not W.is_cuda else W], fp8.SCALE_E8M0)
    y = fp8.batched_gemm_a8w8_mxscale((qa, sa), (qw, sw))
    oqa, osa = oracle.quantize_block_e8m0(X.cpu())
    oqw, osw = oracle.quantize_weight_block(W.cpu(), 1)
    assert_gemm_all_rows(y, oqa, oracle.e8m0_value(osa), oqw, oracle.e8m0_value(osw),
                         oracle.GRAN_BLOCK, what=what)
    return y


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
    rows = np.arange(T)
    oq, os_, _ = oracle.inverse_rope_group_quant(o, pos, cos, sin, synth.ROPE_DIM)
    oqw, osw = oracle.quantize_weight_block(W.reshape(G * N, K), 1)
    ref = oracle.batched_mx_gemm(oq.reshape(-1, G, K), oqw.reshape(G, N, K),
                                 os_.reshape(-1, G, K // 128), osw.reshape(G, N // 128, -1))
    got = y[torch.as_tensor(rows, device=dev())].reshape(rows.size * G, N)
    assert_rows_close(got, ref.reshape(rows.size * G, N), what="rope -> mx gemm")


def test_mx_batched_ragged_rows_full_tiles():
    """Batched MX GEMM on the ping-pong kernel (N a multiple of 256): 300
    tokens leave a 44-row last tile in every group, K = 640 is 5 K steps.
    Every output row of every group against the oracle."""
    M, B, N, K = 300, 3, 512, 640
    say(f"batched MX GEMM M={M} B={B} N={N} K={K}, ragged row tiles")
    X = synth.act_col_outliers(M * B, K, seed=93)
    W = synth.normal_bf16((B * N, K), seed=94, std=0.02)
    qa, sa = fp8.quantize_block_e8m0(X.to(dev()))
    (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_E8M0)
    y = fp8.batched_gemm_a8w8_mxscale((qa.view(M, B, K), sa.view(M, B, K // 128)),
                                      (qw.view(B, N, K), sw.view(B, N // 128, K // 128)))
    oqa, osa = oracle.quantize_block_e8m0(X)
    oqw, osw = oracle.quantize_weight_block(W, 1)
    ref = oracle.batched_mx_gemm(oqa.reshape(M, B, K), oqw.reshape(B, N, K),
                                 osa.reshape(M, B, K // 128), osw.reshape(B, N // 128, K // 128))
    assert_rows_close(y.view(M * B, N), ref.reshape(M * B, N), what="batched mx ragged")


def test_output_projection_full_size():
    """The output projection at the workload size: inverse RoPE + E8M0 group
    quant of o [8192, 64, 128] as 8 groups of 1024, per-group weights
    [8, 1024, 1024] re-quantized with E8M0 scales, the batched MX GEMM.
    Every output row of every group against the oracle's fp64 product of its
    own codes (the quantizer is bit-exact in its own full-size test)."""
    T, G, N = synth.ROPE_TOKENS, synth.ROPE_GROUPS, synth.ROPE_OUT
    K = synth.ROPE_HEADS * synth.ROPE_HEAD_DIM // G
    say(f"output projection T={T} groups={G} N={N} K={K}, every row")
    o, pos = synth.rope_inputs(T, seed=46)
    cos, sin = synth.rope_cache()
    W = synth.normal_bf16((G * N, K), seed=47, std=0.02)
    qa, sa = fp8.inverse_rope_group_quant(o.to(dev()), torch.as_tensor(pos, device=dev()),
                                          torch.as_tensor(cos, device=dev()),
                                          torch.as_tensor(sin, device=dev()), G)
    (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_E8M0)
    y = fp8.batched_gemm_a8w8_mxscale((qa, sa), (qw.view(G, N, K), sw.view(G, N // 128, -1)))
    oq, os_, _ = oracle.inverse_rope_group_quant(o, pos, cos, sin, synth.ROPE_DIM)
    oq, os_ = oq.reshape(T, G, K), os_.reshape(T, G, K // 128)
    oqw, osw = oracle.quantize_weight_block(W, 1)
    oqw, osw = oqw.reshape(G, N, K), osw.reshape(G, N // 128, K // 128)
    for g in range(G):
        assert_gemm_all_rows(y[:, g, :], oq[:, g, :], oracle.e8m0_value(os_[:, g, :]), oqw[g],
                             oracle.e8m0_value(osw[g]), oracle.GRAN_BLOCK,
                             what=f"output projection group {g}")


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
    say(f"MX GEMM stream-K 256-row tiles {M}x{N}x{K}, every row")
    X = synth.act_col_outliers(M, K, seed=M + N + 11)
    W = synth.weight(N, K, seed=N + K + 13)
    y = _mx_check(X, W, f"mx dk {M}x{N}x{K}")
    y2, _ = _mx_pipeline(X, W, rows=[0])
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))  # fixed-order reduce


@pytest.mark.parametrize("name", ["gate_up", "down"])
def test_mx_dense_full_size(name):
    N, K = synth.DENSE_SHAPES[name]
    M = 8192
    say(f"MX GEMM {name} M={M} ({M}x{N}x{K}), every row")
    X, W = synth.dense_linear(name, M, seed=13)
    _mx_check(X, W, f"mx {name}")


def _sweep_shapes(seed: int, n: int):
    """Seeded (M, N, K) triples: M over 1..1400 with the tile edges 127, 128,
    129, 255, 256, 257, 1023, 1024, 1025 mixed in; N and K multiples of 128
    up to 3072 (N with an odd count of 128-column halves as often as not)."""
    rng = np.random.default_rng(seed)
    edges = [1, 127, 128, 129, 255, 256, 257, 1023, 1024, 1025]
    out = []
    for i in range(n):
        M = int(edges[i]) if i < len(edges) else int(rng.integers(1, 1401))
        N = 128 * int(rng.integers(1, 25))
        K = 128 * int(rng.integers(1, 25))
        out.append((M, N, K))
    return out


@pytest.mark.parametrize("gran", ["block", "row", "mx"])
def test_random_shape_sweep(gran):
    """24 seeded shapes per scale form, the kernel choice left to the
    launcher (stream-K, 256-row tiles, whole tiles, the ping-pong kernel,
    128-column tails): every output row of each against the oracle."""
    for i, (M, N, K) in enumerate(_sweep_shapes({"block": 11, "row": 12, "mx": 13}[gran], 24)):
        say(f"{gran} GEMM sweep {i}: {M}x{N}x{K}")
        X = synth.act_col_outliers(M, K, seed=1000 + i)
        W = synth.weight(N, K, seed=2000 + i)
        if gran == "block":
            _block_check(X, W, f"sweep block {M}x{N}x{K}")
        elif gran == "row":
            _row_check(X, W, f"sweep row {M}x{N}x{K}")
        else:
            _mx_check(X, W, f"sweep mx {M}x{N}x{K}")


def test_grouped_random_routing_sweep():
    """Grouped GEMM over seeded routings: 1 to 40 experts, counts from 0 to
    600 rows (empty experts, single rows, 256-row edges), N and K multiples
    of 128; every routed row against the per-expert oracle product."""
    rng = np.random.default_rng(21)
    for i in range(8):
        E = int(rng.integers(1, 41))
        counts = rng.integers(0, 601, size=E)
        if i % 2 == 0:
            counts[rng.integers(0, E)] = 0
            counts[rng.integers(0, E)] = 256
        T = int(counts.sum())
        if T == 0:
            counts[0] = 1
            T = 1
        N = 128 * int(rng.integers(1, 17))
        K = 128 * int(rng.integers(1, 17))
        offsets = np.zeros(E + 1, np.int32)
        offsets[1:] = np.cumsum(counts)
        say(f"grouped GEMM sweep {i}: E={E} T={T} N={N} K={K}")
        A = synth.act_col_outliers(T, K, seed=3000 + i)
        W = synth.normal_bf16((E * N, K), seed=4000 + i, std=0.02)
        qa, sa = fp8.quantize_block(A.to(dev()))
        (qw, sw), = fp8.requantize_weights([W.to(dev())], fp8.SCALE_F32)
        y = fp8.grouped_gemm_a8w8_scaled((qa, sa), (qw.view(E, N, K), sw.view(E, N // 128, K // 128)),
                                         torch.as_tensor(offsets, device=dev()))
        oqa, osa = oracle.quantize_block(A)
        oqw, osw = oracle.quantize_weight_block(W, 0)
        oqw, osw = oqw.reshape(E, N, K), osw.reshape(E, N // 128, K // 128)
        for e in range(E):
            r0, r1 = int(offsets[e]), int(offsets[e + 1])
            if r1 > r0:
                assert_gemm_all_rows(y[r0:r1], oqa[r0:r1], osa[r0:r1], oqw[e], osw[e],
                                     oracle.GRAN_BLOCK, what=f"sweep {i} expert {e}")


def test_layer_chain_in_graph_capture():
    """One captured graph runs a chain of the library's launches: 1x128 quant
    -> block GEMM on the large-M kernel, 1x128 quant -> decode-size block GEMM
    (stream-K with its reduce, workspace from the graph pool), RMSNorm +
    per-token quant -> row-scaled GEMM.  Every replay, with eager work and
    synchronizations between, is bitwise equal to the same chain run eagerly."""
    say("layer chain captured in a HIP graph, 3 replays")
    M, Md, K, N1, N2 = 1024, 256, 2048, 2048, 1536
    x = synth.act_col_outliers(M, K, seed=81).to(dev())
    xd = synth.act_col_outliers(Md, K, seed=82).to(dev())
    h = synth.normal_bf16((M, K), seed=83).to(dev())
    gamma = synth.normal_bf16((K,), seed=84, std=0.5).to(dev())
    (qw1, sw1), = fp8.requantize_weights([synth.weight(N1, K, seed=85).to(dev())], fp8.SCALE_F32)
    qw2, sw2 = fp8.quantize_token(synth.weight(N2, K, seed=86).to(dev()))
    bufs = {
        "qa": torch.empty((M, K), dtype=torch.uint8, device=dev()),
        "sa": torch.empty((M, K // 128), dtype=torch.float32, device=dev()),
        "qd": torch.empty((Md, K), dtype=torch.uint8, device=dev()),
        "sd": torch.empty((Md, K // 128), dtype=torch.float32, device=dev()),
        "q2": torch.empty((M, K), dtype=torch.uint8, device=dev()),
        "s2": torch.empty((M,), dtype=torch.float32, device=dev()),
        "y1": torch.empty((M, N1), dtype=torch.bfloat16, device=dev()),
        "yd": torch.empty((Md, N1), dtype=torch.bfloat16, device=dev()),
        "y2": torch.empty((M, N2), dtype=torch.bfloat16, device=dev()),
    }

    def chain(b):
        fp8.quantize_block(x, out=(b["qa"], b["sa"]))
        fp8.gemm_a8w8_scaled((b["qa"], b["sa"]), (qw1, sw1), fp8.GRAN_BLOCK, out=b["y1"])
        fp8.quantize_block(xd, out=(b["qd"], b["sd"]))
        fp8.gemm_a8w8_scaled((b["qd"], b["sd"]), (qw1, sw1), fp8.GRAN_BLOCK, out=b["yd"])
        fp8.rmsnorm_quant(h, gamma, 1e-6, 0, out=(b["q2"], b["s2"]))
        fp8.gemm_a8w8_scaled((b["q2"], b["s2"]), (qw2, sw2), fp8.GRAN_ROW, out=b["y2"])

    chain(bufs)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in bufs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(bufs)
    for rep in range(3):
        for v in bufs.values():
            v.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in bufs:
            a, b = bufs[k], eager[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), f"replay {rep}: {k} differs from the eager chain"
        _ = fp8.gemm_a8w8_scaled((eager["qd"], eager["sd"]), (qw1, sw1), fp8.GRAN_BLOCK)
        torch.cuda.synchronize()
    oqa, osa = oracle.quantize_block(x.cpu())
    oqw, osw = oracle.quantize_weight_block(synth.weight(N1, K, seed=85), 0)
    rows = [0, 511, 1023]
    ref = oracle.gemm(oqa[rows], oqw, osa[rows], osw, oracle.GRAN_BLOCK)
    assert_rows_close(eager["y1"], ref, rows=rows, what="chain y1")
