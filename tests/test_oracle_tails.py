"""Pins of the oracle GEMM and the operand generator when K is not a multiple
of 128 (a partial last K-block with its own scales; the K tail the FP8 kernel
write-up, demingchina.com/news/60142, section 6, hunts bugs in) and N is not
a multiple of 8.  CPU only.

They tie the tail handling to things other than the oracle itself: exact
rational brute force, the zero-padding identity (padding K with zero codes
up to a multiple of 128 changes nothing), a one-block textbook product, the
generator's partial-block scales, and a planted slip that drops the tail."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import blockscaled as OB
from moe_grouped_gemm_block_amd import inputs as I

FIN4 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
U53 = 2.0 ** -53


def codes(rng, shape):
    return FIN4[rng.integers(0, len(FIN4), shape)]


def exact(A, sA, B, sB):
    tab = [Fraction(float(v)) if np.isfinite(v) else None for v in oracle.decode_table()]
    M, K = A.shape
    N = B.shape[0]
    C = [[Fraction(0)] * N for _ in range(M)]
    mass = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            for k in range(K):
                t = (tab[A[i, k]] * Fraction(float(sA[i // 128, k // 128]))
                     * tab[B[j, k]] * Fraction(float(sB[j // 128, k // 128])))
                C[i][j] += t
                mass[i][j] += abs(t)
    return C, mass


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 16, 0), (4, 3, 144, 1), (2, 7, 272, 2), (3, 2, 40, 3)])
def test_brute_force_k_tail(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A, B = codes(rng, (M, K)), codes(rng, (N, K))
    Kb = -(-K // 128)
    sA = np.exp2(rng.uniform(-10, 10, (1, Kb))).astype(np.float32)
    sB = np.exp2(rng.uniform(-10, 10, (1, Kb))).astype(np.float32)
    C, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    Ce, me = exact(A, sA, B, sB)
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(float(C[i, j])) - Ce[i][j])
            assert err <= Fraction(2 * Kb + 1) * Fraction(U53) * me[i][j], (i, j)


@pytest.mark.parametrize("K", [16, 112, 144, 400, 1040])
def test_zero_padding_k_changes_nothing(K):
    """Padding A and B with zero codes up to a multiple of 128 (same scales)
    gives the same C bit for bit: the tail block's partial is exact either way."""
    rng = np.random.default_rng(K)
    M, N = 9, 11
    A, B = codes(rng, (M, K)), codes(rng, (N, K))
    Kb = -(-K // 128)
    sA = np.exp2(rng.uniform(-6, 6, (1, Kb))).astype(np.float32)
    sB = np.exp2(rng.uniform(-6, 6, (1, Kb))).astype(np.float32)
    Kp = 128 * Kb
    Ap = np.zeros((M, Kp), np.uint8)
    Bp = np.zeros((N, Kp), np.uint8)
    Ap[:, :K], Bp[:, :K] = A, B
    C, m = oracle.gemm_blockscaled(A, sA, B, sB)
    Cp, mp = oracle.gemm_blockscaled(Ap, sA, Bp, sB)
    np.testing.assert_array_equal(C, Cp)
    np.testing.assert_array_equal(m, mp)


def test_single_partial_block_is_a_scaled_textbook_product():
    rng = np.random.default_rng(5)
    A, B = codes(rng, (6, 48)), codes(rng, (10, 48))
    sA = np.array([[0.25]], np.float32)
    sB = np.array([[8.0]], np.float32)
    C, _ = oracle.gemm_blockscaled(A, sA, B, sB)
    np.testing.assert_array_equal(C, 2.0 * (oracle.decode(A) @ oracle.decode(B).T))


def test_grouped_k_tail_is_per_expert_dense():
    rng = np.random.default_rng(6)
    offs = np.array([0, 128, 256], np.int64)
    K, N = 176, 9
    A = codes(rng, (256, K))
    sA = np.exp2(rng.uniform(-4, 4, (2, 2))).astype(np.float32)
    B = codes(rng, (2, N, K))
    sB = np.exp2(rng.uniform(-4, 4, (2, 1, 2))).astype(np.float32)
    C, _ = oracle.grouped_gemm(A, sA, B, sB, offs)
    for e in range(2):
        Ce, _ = oracle.gemm_blockscaled(A[128 * e:128 * e + 128], sA[e:e + 1], B[e], sB[e])
        np.testing.assert_array_equal(C[128 * e:128 * e + 128], Ce)


def test_generator_partial_k_block_scales():
    """The generator's scale of a partial K-block is amax / 448 over that block's columns only."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((130, 200)).astype(np.float32)
    x[:, 128:] *= 10.0
    s = I.block_scales(x)
    assert s.shape == (2, 2)
    for rb in range(2):
        for kb in range(2):
            blk = np.abs(x[128 * rb:128 * rb + 128, 128 * kb:128 * kb + 128])
            assert s[rb, kb] == np.float32(blk.max()) / np.float32(448.0)
    q, s2 = I.quantize(x)
    assert q.shape == x.shape and np.array_equal(s, s2)
    dec = oracle.decode(q) * np.repeat(np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:130, :200]
    # every value within half an E4M3 step (relative 2^-4) or the subnormal spacing
    assert np.all(np.abs(dec - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * np.repeat(
        np.repeat(s.astype(np.float64), 128, 0), 128, 1)[:130, :200]))


def test_planted_dropped_tail_is_caught(monkeypatch):
    """An oracle that ignores the partial last K-block fails the brute force."""
    real = OB.gemm_blockscaled

    def slipped(A, sA, B, sB, rows=None, cols=None, a_fmt="e4m3", b_fmt="e4m3", sa_rows=128):
        Kf = A.shape[1] // 128 * 128
        return real(A[:, :Kf], sA[:, :Kf // 128], B[:, :Kf], sB[:, :Kf // 128], rows, cols, a_fmt, b_fmt, sa_rows)

    monkeypatch.setattr(oracle, "gemm_blockscaled", slipped)
    with pytest.raises(AssertionError):
        test_brute_force_k_tail(4, 3, 144, 1)
