"""Pins for the oracle's dequantize-then-fp64 GEMM and grouped GEMM (CPU only).

Fixed independently by: exact rational sums on tiny shapes (every product of a
code value and a scale is a dyadic rational), a one-hot activation row that
must return decoded weight columns, scale-indexing probes (doubling one scale
doubles exactly that slab's contribution), homogeneity in the scales, and for
the grouped form reduction to per-expert dense products (empty experts
included).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle


def _rand_codes(rng, shape):
    q = rng.integers(0, 256, size=shape, dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38  # no NaN codes
    return q


def _exact_dot(qa_row, sa_row, qw_row, sw_row, gran, tab):
    K = qa_row.size
    total = Fraction(0)
    for k in range(K):
        if gran == oracle.GRAN_BLOCK:
            sa = Fraction(float(sa_row[k // 128]))
            sw = Fraction(float(sw_row[k // 128]))
        else:
            sa = Fraction(float(sa_row))
            sw = Fraction(float(sw_row))
        total += Fraction(tab[qa_row[k]]) * sa * Fraction(tab[qw_row[k]]) * sw
    return total


@pytest.mark.parametrize("gran", [oracle.GRAN_BLOCK, oracle.GRAN_ROW])
def test_tiny_gemm_against_exact_rationals(gran):
    rng = np.random.default_rng(40 + gran)
    tab = oracle.decode_table()
    M, N, K = 3, 256, 256
    qa, qw = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    if gran == oracle.GRAN_BLOCK:
        sa = rng.uniform(1e-3, 1.0, (M, K // 128)).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, (N // 128, K // 128)).astype(np.float32)
    else:
        sa = rng.uniform(1e-3, 1.0, M).astype(np.float32)
        sw = rng.uniform(1e-4, 1e-2, N).astype(np.float32)
    Y = oracle.gemm(qa, qw, sa, sw, gran)
    for m in range(M):
        for n in (0, 1, 127, 128, 200, 255):
            swr = sw[n // 128] if gran == oracle.GRAN_BLOCK else sw[n]
            ex = _exact_dot(qa[m], sa[m], qw[n], swr, gran, tab)
            assert abs(Fraction(Y[m, n]) - ex) <= abs(ex) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 80)


def test_one_hot_row_returns_weight_column():
    rng = np.random.default_rng(1)
    tab = oracle.decode_table()
    N, K = 256, 384
    qw = _rand_codes(rng, (N, K))
    sw = np.ones((N // 128, K // 128), np.float32)
    qa = np.zeros((K, K), np.uint8)
    qa[np.arange(K), np.arange(K)] = 0x38  # 1.0
    sa = np.ones((K, K // 128), np.float32)
    Y = oracle.gemm(qa, qw, sa, sw, oracle.GRAN_BLOCK)
    assert np.array_equal(Y, tab[qw].T)


def test_scale_indexing_probes_and_homogeneity():
    rng = np.random.default_rng(2)
    M, N, K = 8, 384, 512
    qa, qw = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sa = rng.uniform(0.5, 2, (M, K // 128)).astype(np.float32)
    sw = rng.uniform(0.5, 2, (N // 128, K // 128)).astype(np.float32)
    Y = oracle.gemm(qa, qw, sa, sw, oracle.GRAN_BLOCK)

    def slab(m_sel, nb, kb):
        # contribution of activation block kb and weight block (nb, kb) alone
        za = np.zeros_like(sa)
        za[:, kb] = sa[:, kb]
        zw = np.zeros_like(sw)
        zw[nb, kb] = sw[nb, kb]
        return oracle.gemm(qa, qw, za, zw, oracle.GRAN_BLOCK)

    # doubling sA[m, kb] adds exactly row m's kb contribution (all n blocks)
    sa2 = sa.copy()
    sa2[3, 2] *= 2
    Y2 = oracle.gemm(qa, qw, sa2, sw, oracle.GRAN_BLOCK)
    add = sum(slab(None, nb, 2) for nb in range(N // 128))
    exp = Y.copy()
    exp[3] += add[3]
    tol = 1e-12 * np.abs(Y).max()
    assert np.allclose(Y2, exp, rtol=0, atol=tol)
    # doubling sW[nb, kb] adds exactly that block's contribution for all rows
    sw2 = sw.copy()
    sw2[1, 3] *= 2
    Y3 = oracle.gemm(qa, qw, sa, sw2, oracle.GRAN_BLOCK)
    exp = Y.copy()
    exp[:, 128:256] += slab(None, 1, 3)[:, 128:256]
    assert np.allclose(Y3, exp, rtol=0, atol=tol)
    assert np.array_equal(Y3[:, :128], Y[:, :128]) and np.array_equal(Y3[:, 256:], Y[:, 256:])
    # homogeneity with a power of two is exact
    assert np.array_equal(oracle.gemm(qa, qw, sa * 4, sw, oracle.GRAN_BLOCK), 4 * Y)


def test_grouped_reduces_to_per_expert_dense():
    rng = np.random.default_rng(3)
    E, N, K = 5, 256, 256
    counts = np.array([3, 0, 7, 0, 2])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = offsets[-1]
    qa, qw = _rand_codes(rng, (T, K)), _rand_codes(rng, (E, N, K))
    sa = rng.uniform(0.5, 2, (T, K // 128)).astype(np.float32)
    sw = rng.uniform(0.5, 2, (E, N // 128, K // 128)).astype(np.float32)
    Y = oracle.grouped_gemm(qa, qw, sa, sw, offsets)
    for e in range(E):
        a, b = offsets[e], offsets[e + 1]
        if a == b:
            continue
        Ye = oracle.gemm(qa[a:b], qw[e], sa[a:b], sw[e], oracle.GRAN_BLOCK)
        # same sums; the fp64 product may block differently for other shapes
        assert np.allclose(Y[a:b], Ye, rtol=0, atol=1e-13 * np.abs(Ye).max())
    rows = np.array([0, 4, 11])
    Yr = oracle.grouped_gemm(qa, qw, sa, sw, offsets, rows=rows)
    assert np.allclose(Yr, Y[rows], rtol=0, atol=1e-13 * np.abs(Y).max())


def test_mx_gemm_against_exact_rationals():
    """E8M0 bytes stand for 2^(b - 127): exact rational sums on a tiny shape."""
    rng = np.random.default_rng(77)
    tab = oracle.decode_table()
    M, N, K = 3, 256, 384
    qa, qw = _rand_codes(rng, (M, K)), _rand_codes(rng, (N, K))
    sa8 = rng.integers(110, 140, (M, K // 128)).astype(np.uint8)
    sw8 = rng.integers(100, 135, (N // 128, K // 128)).astype(np.uint8)
    Y = oracle.mx_gemm(qa, qw, sa8, sw8)
    for m in range(M):
        for n in (0, 5, 127, 128, 255):
            ex = Fraction(0)
            for k in range(K):
                ex += (Fraction(tab[qa[m, k]]) * Fraction(2) ** (int(sa8[m, k // 128]) - 127) *
                       Fraction(tab[qw[n, k]]) * Fraction(2) ** (int(sw8[n // 128, k // 128]) - 127))
            assert abs(Fraction(Y[m, n]) - ex) <= abs(ex) * Fraction(1, 2 ** 40) + Fraction(1, 2 ** 200)


def test_batched_mx_gemm_equals_block_diagonal_dense():
    """Batch b of [M, B, K] x [B, N, K] -> [M, B, N] equals the dense product of
    A laid out as [M, B*K] with a block-diagonal [B*N, B*K] weight (zero codes
    off the diagonal)."""
    rng = np.random.default_rng(78)
    M, B, N, K = 5, 3, 128, 256
    qa = _rand_codes(rng, (M, B, K))
    qw = _rand_codes(rng, (B, N, K))
    sa8 = rng.integers(115, 135, (M, B, K // 128)).astype(np.uint8)
    sw8 = rng.integers(110, 130, (B, N // 128, K // 128)).astype(np.uint8)
    Y = oracle.batched_mx_gemm(qa, qw, sa8, sw8)
    A = qa.reshape(M, B * K)
    SA = sa8.reshape(M, B * K // 128)
    W = np.zeros((B * N, B * K), np.uint8)
    SW = np.full((B * N // 128, B * K // 128), 127, np.uint8)
    for b in range(B):
        W[b * N:(b + 1) * N, b * K:(b + 1) * K] = qw[b]
        SW[b * N // 128:(b + 1) * N // 128, b * K // 128:(b + 1) * K // 128] = sw8[b]
    D = oracle.mx_gemm(A, W, SA, SW).reshape(M, B, N)
    assert np.allclose(Y, D, rtol=1e-12, atol=0.0)
    Y1 = oracle.batched_mx_gemm(qa[:, 1:2], qw[1:2], sa8[:, 1:2], sw8[1:2])
    assert np.array_equal(Y1[:, 0], oracle.mx_gemm(np.ascontiguousarray(qa[:, 1]), qw[1],
                                                    np.ascontiguousarray(sa8[:, 1]), sw8[1]))
