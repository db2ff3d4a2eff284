"""Pins of the oracle GEMM with one A scale per row and 128-wide K-block
(sa_rows = 1, the 1 x 128 granularity of the FP8 kernel write-up,
demingchina.com/news/60142, section 5.2 table).  CPU only.

They tie the per-row indexing to things other than the oracle itself: exact
rational brute force, the 128 x 128 case it must reduce to when the scales of
a 128-row block agree, the diagonal identity C = diag(s) C_1 on one K-block,
the grouped form against per-expert dense products, and planted slips."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import blockscaled as OB

FIN4 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
U53 = 2.0 ** -53


def codes(rng, shape):
    return FIN4[rng.integers(0, len(FIN4), shape)]


def exact_rowscaled(A, sA, B, sB):
    """C[i][j] = sum_kb sA[i, kb] sB[j // 128, kb] sum_k dec(A) dec(B), in rationals."""
    tab = [Fraction(float(v)) if np.isfinite(v) else None for v in oracle.decode_table()]
    M, K = A.shape
    N = B.shape[0]
    C = [[Fraction(0)] * N for _ in range(M)]
    mass = [[Fraction(0)] * N for _ in range(M)]
    for kb in range(K // 128):
        for i in range(M):
            for j in range(N):
                s = Fraction(float(sA[i, kb])) * Fraction(float(sB[j // 128, kb]))
                p = sum(tab[A[i, k]] * tab[B[j, k]] for k in range(128 * kb, 128 * kb + 128))
                q = sum(abs(tab[A[i, k]] * tab[B[j, k]]) for k in range(128 * kb, 128 * kb + 128))
                C[i][j] += s * p
                mass[i][j] += s * q
    return C, mass


@pytest.mark.parametrize("M,N,K,seed", [(5, 4, 128, 0), (7, 3, 384, 1), (3, 130, 256, 2)])
def test_brute_force_row_scales(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A, B = codes(rng, (M, K)), codes(rng, (N, K))
    sA = np.exp2(rng.uniform(-12, 12, (M, K // 128))).astype(np.float32)
    sB = np.exp2(rng.uniform(-12, 12, (-(-N // 128), K // 128))).astype(np.float32)
    C, mass = oracle.gemm_blockscaled(A, sA, B, sB, sa_rows=1)
    Ce, me = exact_rowscaled(A, sA, B, sB)
    Kb = K // 128
    for i in range(M):
        for j in range(N):
            # E4M3 block partials are exact in float64; Kb scaled adds round
            err = abs(Fraction(float(C[i, j])) - Ce[i][j])
            assert err <= Fraction(2 * Kb + 1) * Fraction(U53) * me[i][j], (i, j)
            assert abs(Fraction(float(mass[i, j])) - me[i][j]) <= Fraction(2 * Kb + 1) * Fraction(U53) * me[i][j]


def test_reduces_to_128x128_when_a_block_shares_its_scale():
    rng = np.random.default_rng(3)
    M, N, K = 300, 140, 384
    A, B = codes(rng, (M, K)), codes(rng, (N, K))
    s128 = np.exp2(rng.uniform(-6, 6, (3, 3))).astype(np.float32)
    sB = np.exp2(rng.uniform(-6, 6, (2, 3))).astype(np.float32)
    s1 = np.repeat(s128, 128, axis=0)[:M]
    C1, m1 = oracle.gemm_blockscaled(A, s1, B, sB, sa_rows=1)
    C128, m128 = oracle.gemm_blockscaled(A, s128, B, sB)
    np.testing.assert_array_equal(C1, C128)
    np.testing.assert_array_equal(m1, m128)


def test_one_k_block_is_a_row_diagonal_scaling():
    """With one K-block, C = diag(sA[:, 0]) C_unit exactly for power-of-two scales."""
    rng = np.random.default_rng(4)
    M, N, K = 37, 20, 128
    A, B = codes(rng, (M, K)), codes(rng, (N, K))
    e = rng.integers(-8, 9, M)
    sA = np.exp2(e).astype(np.float32)[:, None]
    one = np.ones((1, 1), np.float32)
    C, _ = oracle.gemm_blockscaled(A, sA, B, one, sa_rows=1)
    Cu, _ = oracle.gemm_blockscaled(A, one, B, one)
    np.testing.assert_array_equal(C, Cu * np.exp2(e)[:, None])
    # and C_unit is the plain product of the decoded operands
    np.testing.assert_array_equal(Cu, oracle.decode(A) @ oracle.decode(B).T)


def test_grouped_row_scales_are_per_expert_dense_products():
    rng = np.random.default_rng(5)
    offs = np.array([0, 128, 128, 384], np.int64)
    G, N, K = 3, 24, 256
    A = codes(rng, (384, K))
    sA = np.exp2(rng.uniform(-5, 5, (384, K // 128))).astype(np.float32)
    B = codes(rng, (G, N, K))
    sB = np.exp2(rng.uniform(-5, 5, (G, 1, K // 128))).astype(np.float32)
    C, _ = oracle.grouped_gemm(A, sA, B, sB, offs, sa_rows=1)
    for e in range(G):
        lo, hi = offs[e], offs[e + 1]
        if hi > lo:
            Ce, _ = oracle.gemm_blockscaled(A[lo:hi], sA[lo:hi], B[e], sB[e], sa_rows=1)
            np.testing.assert_array_equal(C[lo:hi], Ce)
    rows = np.array([0, 127, 200, 383])
    Cs, _ = oracle.grouped_gemm(A, sA, B, sB, offs, rows=rows, sa_rows=1)
    np.testing.assert_array_equal(Cs, C[rows])


def test_bad_sa_rows_rejected():
    A = np.zeros((2, 128), np.uint8)
    s = np.ones((2, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.gemm_blockscaled(A, s, A, s, sa_rows=64)


def test_planted_block_index_slip_is_caught(monkeypatch):
    """An oracle that kept indexing sA by i // 128 for per-row scales fails the brute force."""
    real = OB.gemm_blockscaled

    def slipped(A, sA, B, sB, rows=None, cols=None, a_fmt="e4m3", b_fmt="e4m3", sa_rows=128):
        M = A.shape[0]
        r = np.arange(M)
        wrong = sA[(r // 128) * 128] if sa_rows == 1 else sA        # row block's first row
        return real(A, wrong, B, sB, rows, cols, a_fmt, b_fmt, sa_rows)

    monkeypatch.setattr(oracle, "gemm_blockscaled", slipped)
    with pytest.raises(AssertionError):
        test_brute_force_row_scales(5, 4, 128, 0)


def test_packed_segments_are_per_expert_dense_products():
    """Segments that start anywhere (no padding rows), per-row A scales: every
    expert's rows are the dense product with that expert's B, and rows of a
    segment never see another expert's weights."""
    rng = np.random.default_rng(6)
    offs = np.array([0, 3, 3, 20, 21, 85], np.int64)          # 3, 0, 17, 1, 64 rows
    G, N, K = 5, 24, 256
    A = codes(rng, (85, K))
    sA = np.exp2(rng.uniform(-5, 5, (85, K // 128))).astype(np.float32)
    B = codes(rng, (G, N, K))
    sB = np.exp2(rng.uniform(-5, 5, (G, 1, K // 128))).astype(np.float32)
    C, _ = oracle.grouped_gemm(A, sA, B, sB, offs, sa_rows=1)
    for e in range(G):
        lo, hi = offs[e], offs[e + 1]
        if hi > lo:
            Ce, _ = oracle.gemm_blockscaled(A[lo:hi], sA[lo:hi], B[e], sB[e], sa_rows=1)
            np.testing.assert_array_equal(C[lo:hi], Ce)
    # brute force on one row of each non-empty segment
    for i in (0, 2, 3, 19, 20, 21, 84):
        e = int(np.searchsorted(offs, i, side="right") - 1)
        Ce, me = exact_rowscaled(A[i:i + 1], sA[i:i + 1], B[e], sB[e])
        for j in range(N):
            err = abs(Fraction(float(C[i, j])) - Ce[0][j])
            assert err <= Fraction(5) * Fraction(U53) * me[0][j], (i, j)


def test_packed_segments_need_row_scales():
    A = np.zeros((10, 128), np.uint8)
    B = np.zeros((2, 8, 128), np.uint8)
    sB = np.ones((2, 1, 1), np.float32)
    with pytest.raises(ValueError):
        oracle.grouped_gemm(A, np.ones((1, 1), np.float32), B, sB, np.array([0, 3, 10]))
