"""Pins of the oracle's E5M2 decode and of the GEMM oracle with E5M2 operands
(CPU only): a library cast (torch.float8_e5m2), the closed form "an E5M2 byte
is the high byte of an IEEE half", the format table of the DeepGEMM FP8
kernel write-up (section 3.1, golden fixture), exact rational brute force with
mixed formats, integer-valued operands, and planted slips."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import blockscaled as OB

FIN5 = np.array([c for c in range(256) if ((c >> 2) & 0x1F) != 0x1F], np.uint8)
FIN4 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
U53 = 2.0 ** -53


def lib_decode5(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return t.view(torch.float8_e5m2).to(torch.float64).numpy()


def lib_decode4(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_e5m2_vs_library():
    ours = oracle.decode_table("e5m2")
    lib = lib_decode5(np.arange(256))
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(ours[ok], lib[ok])
    assert np.isinf(ours[0x7C]) and ours[0x7C] > 0 and np.isinf(ours[0xFC]) and ours[0xFC] < 0
    assert np.signbit(ours[0x80]) and ours[0x80] == 0


def test_decode_e5m2_is_the_high_byte_of_a_half():
    halves = (np.arange(256, dtype=np.uint16) << 8).view(np.float16).astype(np.float64)
    ours = oracle.decode_table("e5m2")
    ok = ~np.isnan(halves)
    assert np.array_equal(np.isnan(ours), ~ok)
    np.testing.assert_array_equal(ours[ok], halves[ok])


def test_decode_e5m2_matches_page_format_table(golden_dir):
    spec = json.load(open(os.path.join(golden_dir, "e4m3_format.json")))["formats"]["E5M2"]
    e_bits, m_bits = spec["exponent_bits"], spec["mantissa_bits"]
    assert spec["sign_bits"] + e_bits + m_bits == 8
    tab = oracle.decode_table("e5m2")
    finite = tab[np.isfinite(tab)]
    assert finite.max() == spec["max_approx"] == 57344
    bias = 2 ** (e_bits - 1) - 1
    assert np.min(np.abs(finite[finite != 0])) == 2.0 ** (1 - bias - m_bits)
    one = np.sort(finite[(finite >= 1) & (finite < 2)])
    np.testing.assert_array_equal(np.diff(one), 2.0 ** -m_bits)


def exact(A, a_dec, sA, B, b_dec, sB):
    M, K = A.shape
    N = B.shape[0]
    Ad, Bd = a_dec(A), b_dec(B)
    Ax = [[Fraction(float(Ad[i, k])) * Fraction(float(sA[i // 128, k // 128])) for k in range(K)]
          for i in range(M)]
    Bx = [[Fraction(float(Bd[j, k])) * Fraction(float(sB[j // 128, k // 128])) for k in range(K)]
          for j in range(N)]
    C = [[sum(Ax[i][k] * Bx[j][k] for k in range(K)) for j in range(N)] for i in range(M)]
    mass = [[sum(abs(Ax[i][k] * Bx[j][k]) for k in range(K)) for j in range(N)] for i in range(M)]
    return C, mass


@pytest.mark.parametrize("a_fmt,b_fmt", [("e5m2", "e5m2"), ("e5m2", "e4m3"), ("e4m3", "e5m2")])
@pytest.mark.parametrize("M,N,K,seed", [(4, 5, 128, 0), (6, 3, 256, 1)])
def test_brute_force_mixed_formats(a_fmt, b_fmt, M, N, K, seed):
    rng = np.random.default_rng(seed)
    fin = {"e5m2": FIN5, "e4m3": FIN4}
    dec = {"e5m2": lib_decode5, "e4m3": lib_decode4}
    A = fin[a_fmt][rng.integers(0, len(fin[a_fmt]), (M, K))]
    B = fin[b_fmt][rng.integers(0, len(fin[b_fmt]), (N, K))]
    sA = np.exp2(rng.uniform(-10, 10, (1, K // 128))).astype(np.float32)
    sB = np.exp2(rng.uniform(-10, 10, (1, K // 128))).astype(np.float32)
    C, mass = oracle.gemm_blockscaled(A, sA, B, sB, a_fmt=a_fmt, b_fmt=b_fmt)
    Ce, me = exact(A, dec[a_fmt], sA, B, dec[b_fmt], sB)
    Kb = K // 128
    for i in range(M):
        for j in range(N):
            # BLAS summation of up to 128 products per block, then Kb + 1 roundings
            err = abs(Fraction(float(C[i, j])) - Ce[i][j])
            assert err <= Fraction(128 * Kb + Kb + 1) * Fraction(U53) * me[i][j], (i, j)


def test_integer_e5m2_operands_exact():
    """Integer-valued E5M2 codes with power-of-two scales: an int64 matmul."""
    tab = oracle.decode_table("e5m2")
    ints = np.array([c for c in range(256) if np.isfinite(tab[c]) and tab[c] == np.round(tab[c])
                     and abs(tab[c]) <= 16], np.uint8)
    rng = np.random.default_rng(3)
    M, N, K = 9, 7, 256
    A = ints[rng.integers(0, len(ints), (M, K))]
    B = ints[rng.integers(0, len(ints), (N, K))]
    ea, eb = rng.integers(-3, 4, (1, 2)), rng.integers(-3, 4, (1, 2))
    sA, sB = np.exp2(ea).astype(np.float32), np.exp2(eb).astype(np.float32)
    C, _ = oracle.gemm_blockscaled(A, sA, B, sB, a_fmt="e5m2", b_fmt="e5m2")
    Ai, Bi = tab[A].astype(np.int64), tab[B].astype(np.int64)
    want = np.zeros((M, N))
    for kb in range(2):
        ks = slice(128 * kb, 128 * kb + 128)
        want += (Ai[:, ks] @ Bi[:, ks].T).astype(np.float64) * 2.0 ** (ea[0, kb] + eb[0, kb])
    np.testing.assert_array_equal(C, want)


def test_default_format_is_e4m3():
    rng = np.random.default_rng(4)
    A = FIN4[rng.integers(0, len(FIN4), (3, 128))]
    B = FIN4[rng.integers(0, len(FIN4), (2, 128))]
    s = np.ones((1, 1), np.float32)
    np.testing.assert_array_equal(oracle.gemm_blockscaled(A, s, B, s)[0],
                                  oracle.gemm_blockscaled(A, s, B, s, a_fmt="e4m3", b_fmt="e4m3")[0])


@pytest.mark.parametrize("slip", ["bias_16", "e4m3_table"])
def test_planted_e5m2_slips_are_caught(monkeypatch, slip):
    tab = oracle.decode_table("e5m2").copy()
    if slip == "bias_16":
        tab = tab / 2.0
    else:
        tab = oracle.decode_table("e4m3").copy()
    monkeypatch.setitem(OB._LUTS, "e5m2", tab)
    with pytest.raises(AssertionError):
        test_brute_force_mixed_formats("e5m2", "e5m2", 4, 5, 128, 0)
