"""Pins of the CPU oracle to facts fixed outside it (CPU only).

Each check is chosen so that a plausible slip in the oracle -- a wrong
exponent bias, flushed subnormals, a dropped K-block, a scale taken from the
wrong block, a transposed operand -- fails at least one of them:

* decode: every byte against a library cast and against the format table
  printed on the DeepGEMM FP8 kernel write-up (section 3.1);
* exact rational brute force on tiny shapes, computed the other way round
  (dequantise every element exactly, then a plain triple loop);
* integer-valued operands with power-of-two block scales, where the product
  is an int64 matmul;
* identity and permutation A, a single 128^3 block (textbook matmul), uniform
  scales (the per-tensor form);
* invariances: consistent K-block reordering, scale homogeneity, swapping
  the roles of A and B, grouped == concatenated per-expert dense.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import blockscaled as OB

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
U53 = 2.0 ** -53


def lib_decode(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def rand_codes(rng, shape):
    return FINITE[rng.integers(0, len(FINITE), size=shape)]


def rand_scales(rng, shape, lo=-12, hi=12):
    return np.exp2(rng.uniform(lo, hi, size=shape)).astype(np.float32)


# --------------------------------------------------------------------------- decode

def test_decode_all_codes_vs_library():
    ours = oracle.decode_table()
    lib = lib_decode(np.arange(256))
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(ours[~nan], lib[~nan])
    # signed zero kept
    assert np.signbit(ours[0x80]) and ours[0x80] == 0


def test_decode_matches_page_format_table(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "e4m3_format.json")))["formats"]["E4M3"]
    e_bits, m_bits = spec["exponent_bits"], spec["mantissa_bits"]
    assert spec["sign_bits"] + e_bits + m_bits == 8
    tab = oracle.decode_table()
    finite = tab[~np.isnan(tab)]
    assert finite.max() == spec["max_approx"] == 448
    # 2^(e+m) magnitudes per sign, one of them NaN
    assert len(np.unique(np.abs(finite))) == 2 ** (e_bits + m_bits) - 1
    bias = 2 ** (e_bits - 1) - 1
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** (1 - bias - m_bits)
    # spacing inside the binade [1, 2) is 2^-m
    one = np.sort(finite[(finite >= 1) & (finite < 2)])
    np.testing.assert_array_equal(np.diff(one), 2.0 ** -m_bits)


# --------------------------------------------------------------------------- brute force

def exact_blockscaled(A, sA, B, sB):
    """Exact rationals: dequantise every element, then a plain triple loop."""
    M, K = A.shape
    N = B.shape[0]
    Ad = lib_decode(A)
    Bd = lib_decode(B)
    Ax = [[Fraction(float(Ad[i, k])) * Fraction(float(sA[i // 128, k // 128]))
           for k in range(K)] for i in range(M)]
    Bx = [[Fraction(float(Bd[j, k])) * Fraction(float(sB[j // 128, k // 128]))
           for k in range(K)] for j in range(N)]
    C = [[sum(Ax[i][k] * Bx[j][k] for k in range(K)) for j in range(N)] for i in range(M)]
    mass = [[sum(abs(Ax[i][k] * Bx[j][k]) for k in range(K)) for j in range(N)] for i in range(M)]
    return C, mass


@pytest.mark.parametrize("M,N,K,seed", [(3, 5, 128, 0), (8, 7, 256, 1), (5, 8, 384, 2),
                                        (130, 2, 256, 3), (2, 131, 384, 4)])
def test_brute_force_exact(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A = rand_codes(rng, (M, K))
    B = rand_codes(rng, (N, K))
    sA = rand_scales(rng, (-(-M // 128), K // 128))
    sB = rand_scales(rng, (-(-N // 128), K // 128))
    C, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    Ce, me = exact_blockscaled(A, sA, B, sB)
    Kb = K // 128
    for i in range(M):
        for j in range(N):
            err = abs(Fraction(float(C[i, j])) - Ce[i][j])
            assert err <= Fraction(Kb + 1) * Fraction(U53) * me[i][j], (i, j)
            assert abs(Fraction(float(mass[i, j])) - me[i][j]) <= Fraction(Kb + 1) * Fraction(U53) * me[i][j]


# --------------------------------------------------------------------------- closed forms

INT_VALUES = np.arange(-16, 17)


def test_integer_operands_power_of_two_scales_exact():
    """Integer E4M3 values |v| <= 16 and 2^e block scales: C * 64 is an int64 matmul."""
    rng = np.random.default_rng(5)
    M, N, K = 200, 136, 512
    Ai = rng.choice(INT_VALUES, size=(M, K))
    Bi = rng.choice(INT_VALUES, size=(N, K))
    to_code = lambda v: torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    A, B = to_code(Ai), to_code(Bi)
    ea = rng.integers(-3, 4, size=(2, 4))
    eb = rng.integers(-3, 4, size=(2, 4))
    sA, sB = np.exp2(ea).astype(np.float32), np.exp2(eb).astype(np.float32)
    At = Ai * (2 ** (np.repeat(np.repeat(ea, 128, 0), 128, 1)[:M] + 3))
    Bt = Bi * (2 ** (np.repeat(np.repeat(eb, 128, 0), 128, 1)[:N] + 3))
    want = (At.astype(np.int64) @ Bt.astype(np.int64).T)
    C, _ = oracle.gemm_blockscaled(A, sA, B, sB)
    np.testing.assert_array_equal(C * 64, want.astype(np.float64))


def test_identity_and_permutation_A():
    rng = np.random.default_rng(6)
    K = N = 256
    B = rand_codes(rng, (N, K))
    sB = rand_scales(rng, (2, 2))
    one = np.uint8(0x38)                                            # E4M3 code of 1.0
    Bdq = lib_decode(B) * np.repeat(np.repeat(sB.astype(np.float64), 128, 0), 128, 1)
    ident = np.where(np.eye(K, dtype=bool), one, np.uint8(0))
    C, _ = oracle.gemm_blockscaled(ident, np.ones((2, 2), np.float32), B, sB)
    np.testing.assert_array_equal(C, Bdq.T)
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.uint8)
    P[np.arange(K), perm] = one
    C, _ = oracle.gemm_blockscaled(P, np.ones((2, 2), np.float32), B, sB)
    np.testing.assert_array_equal(C, Bdq.T[perm])


def test_single_block_is_textbook_matmul():
    rng = np.random.default_rng(7)
    A = rand_codes(rng, (128, 128))
    B = rand_codes(rng, (128, 128))
    sA = np.array([[0.0123]], np.float32)
    sB = np.array([[3.5e-3]], np.float32)
    want = (torch.from_numpy(lib_decode(A)) @ torch.from_numpy(lib_decode(B)).T).numpy()
    want = want * (np.float64(sA[0, 0]) * np.float64(sB[0, 0]))
    C, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    assert np.all(np.abs(C - want) <= 2 * U53 * mass)


def test_uniform_scales_reduce_to_per_tensor_form():
    rng = np.random.default_rng(8)
    M, N, K = 160, 200, 640
    A, B = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    a, b = np.float32(0.37), np.float32(1.9e-4)
    C, mass = oracle.gemm_blockscaled(A, np.full((2, 5), a), B, np.full((2, 5), b))
    want = np.float64(a) * np.float64(b) * (lib_decode(A) @ lib_decode(B).T)
    assert np.all(np.abs(C - want) <= 8 * U53 * mass)


# --------------------------------------------------------------------------- invariances

def test_kblock_reordering_invariance():
    rng = np.random.default_rng(9)
    M, N, K = 130, 70, 768
    A, B = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sA, sB = rand_scales(rng, (2, 6)), rand_scales(rng, (1, 6))
    C, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    p = rng.permutation(6)
    cols = np.concatenate([np.arange(k * 128, (k + 1) * 128) for k in p])
    C2, _ = oracle.gemm_blockscaled(A[:, cols], sA[:, p], B[:, cols], sB[:, p])
    assert np.all(np.abs(C - C2) <= 16 * U53 * mass)
    # and a K-block really matters: dropping one changes the result
    C3, _ = oracle.gemm_blockscaled(A[:, :640], sA[:, :5], B[:, :640], sB[:, :5])
    assert np.abs(C - C3).max() > 0


def test_scale_homogeneity_exact():
    rng = np.random.default_rng(10)
    A, B = rand_codes(rng, (64, 384)), rand_codes(rng, (96, 384))
    sA, sB = rand_scales(rng, (1, 3), -4, 4), rand_scales(rng, (1, 3), -4, 4)
    C, _ = oracle.gemm_blockscaled(A, sA, B, sB)
    C2, _ = oracle.gemm_blockscaled(A, sA * np.float32(8.0), B, sB)
    np.testing.assert_array_equal(C2, 8.0 * C)
    # scaling one A row block touches exactly those rows
    sA2 = sA.copy()
    sA2[0, 1] *= 2
    C3, _ = oracle.gemm_blockscaled(A, sA2, B, sB)
    assert not np.array_equal(C3, C)


def test_swapping_operands_transposes():
    rng = np.random.default_rng(11)
    M, N, K = 150, 260, 384
    A, B = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sA, sB = rand_scales(rng, (2, 3)), rand_scales(rng, (3, 3))
    C, _ = oracle.gemm_blockscaled(A, sA, B, sB)
    Ct, _ = oracle.gemm_blockscaled(B, sB, A, sA)
    np.testing.assert_array_equal(Ct, C.T)


def test_row_col_subsets_match_full():
    rng = np.random.default_rng(12)
    A, B = rand_codes(rng, (300, 256)), rand_codes(rng, (200, 256))
    sA, sB = rand_scales(rng, (3, 2)), rand_scales(rng, (2, 2))
    C, m = oracle.gemm_blockscaled(A, sA, B, sB)
    r = np.array([0, 127, 128, 255, 299])
    c = np.array([5, 130, 199])
    Cs, ms = oracle.gemm_blockscaled(A, sA, B, sB, rows=r, cols=c)
    np.testing.assert_array_equal(Cs, C[np.ix_(r, c)])
    np.testing.assert_array_equal(ms, m[np.ix_(r, c)])


def test_grouped_equals_per_expert_dense():
    rng = np.random.default_rng(13)
    G, N, K = 4, 136, 256
    seg = np.array([256, 0, 128, 384])                               # one empty expert
    off = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    Mt = int(off[-1])
    A = rand_codes(rng, (Mt, K))
    A[200:256] = 0                                                   # padding rows
    sA = rand_scales(rng, (Mt // 128, 2))
    B = rand_codes(rng, (G, N, K))
    sB = rand_scales(rng, (G, 2, 2))
    C, mass = oracle.grouped_gemm(A, sA, B, sB, off)
    for e in range(G):
        lo, hi = off[e], off[e + 1]
        if lo == hi:
            continue
        Ce, _ = oracle.gemm_blockscaled(A[lo:hi], sA[lo // 128:hi // 128], B[e], sB[e])
        np.testing.assert_array_equal(C[lo:hi], Ce)
    assert np.all(C[200:256] == 0)
    # G = 1 reduces to dense
    C1, _ = oracle.grouped_gemm(A, sA, B[:1], sB[:1], np.array([0, Mt], np.int32))
    Cd, _ = oracle.gemm_blockscaled(A, sA, B[0], sB[0])
    np.testing.assert_array_equal(C1, Cd)
    # sampled rows agree with the full result
    r = np.array([0, 255, 256, 383, 384, 767])
    Cs, _ = oracle.grouped_gemm(A, sA, B, sB, off, rows=r, cols=np.array([0, 135]))
    np.testing.assert_array_equal(Cs, C[np.ix_(r, [0, 135])])


# --------------------------------------------------------------------------- planted slips

@pytest.mark.parametrize("slip", ["bias_off_by_one", "flush_subnormals"])
def test_pins_catch_planted_decode_slips(monkeypatch, slip):
    """A wrong decode table planted in the oracle must fail the brute force."""
    tab = oracle.decode_table().copy()
    if slip == "bias_off_by_one":
        tab = tab * 2.0
    else:
        sub = ((np.arange(256) >> 3) & 0xF) == 0
        tab[sub] = 0.0
    monkeypatch.setitem(OB._LUTS, "e4m3", tab)
    with pytest.raises(AssertionError):
        test_brute_force_exact(8, 7, 256, 1)


def test_pins_catch_planted_scale_index_slip(monkeypatch):
    """Taking B's scale from A's row block (a plausible index slip) must fail."""
    real = OB.gemm_blockscaled

    def slipped(A, sA, B, sB, rows=None, cols=None):
        return real(A, sA, B, sA[: sB.shape[0]] if sA.shape[0] >= sB.shape[0] else sB, rows, cols)

    monkeypatch.setattr(oracle, "gemm_blockscaled", slipped)
    with pytest.raises(AssertionError):
        test_brute_force_exact(130, 2, 256, 3)
