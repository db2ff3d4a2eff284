"""Parity of the GEMMs with E5M2 operands (through the C-ABI) with the CPU
oracle.  Needs a GPU.  Same bar as the E4M3 path: |C_gpu - C_ref| <=
1e-5 * mass + 1e-6 (FP32 out), plus 2^-8 |C_ref| for BF16 out."""
import sys

import numpy as np
import pytest
import torch

import parity_log

import oracle
from moe_grouped_gemm_block_amd import dg
from moe_grouped_gemm_block_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
COMBOS = [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_dense(p):
    C = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), p.out_dtype, a_fmt=p.a_fmt, b_fmt=p.b_fmt)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def check(Cg, Cr, mass, out_dtype, what):
    bound = oracle.tolerance(Cr, mass, out_dtype)
    err = np.abs(Cg - Cr)
    log(f"  {what}: max err/bound = {float((err / bound).max()):.3g}")
    parity_log.record(f"e5m2 {what}", float((err / bound).max()))
    assert np.all(np.isfinite(Cg))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
@pytest.mark.parametrize("M,N,K", [(63, 136, 128), (129, 264, 384), (256, 520, 256)])
def test_dense_small(M, N, K, a_fmt, b_fmt, out):
    log(f"e5m2 dense {M}x{N}x{K} {a_fmt}x{b_fmt} {out}")
    p = I.dense_problem(M, N, K, seed=M + N + K, out_dtype=out, block_log2_range=3.0,
                        a_fmt=a_fmt, b_fmt=b_fmt)
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, a_fmt=a_fmt, b_fmt=b_fmt)
    check(run_dense(p), Cr, mass, out, f"{M}x{N}x{K} {a_fmt}x{b_fmt} {out}")


@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
@pytest.mark.parametrize("M,N,K", [(17, 12304, 384), (64, 520, 256)])
def test_few_rows(M, N, K, a_fmt, b_fmt):
    log(f"e5m2 few rows {M}x{N}x{K} {a_fmt}x{b_fmt}")
    p = I.dense_problem(M, N, K, seed=M + N, out_dtype="bf16", outlier_frac=0.01, a_fmt=a_fmt, b_fmt=b_fmt)
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, a_fmt=a_fmt, b_fmt=b_fmt)
    check(run_dense(p), Cr, mass, "bf16", f"few rows {M}x{N}x{K} {a_fmt}x{b_fmt}")


@pytest.mark.parametrize("a_fmt,b_fmt", COMBOS)
def test_grouped(a_fmt, b_fmt):
    log(f"e5m2 grouped {a_fmt}x{b_fmt}")
    rng = np.random.default_rng(3)
    counts, N, K = [300, 0, 130, 512], 264, 384
    padded = [-(-c // 128) * 128 for c in counts]
    offs = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    A = np.zeros((int(offs[-1]), K), np.float32)
    for e, c in enumerate(counts):
        A[offs[e]:offs[e] + c] = rng.standard_normal((c, K), dtype=np.float32)
    qA, sA = I.quantize(A, fmt=a_fmt)
    qB = np.empty((len(counts), N, K), np.uint8)
    sB = np.empty((len(counts), -(-N // 128), K // 128), np.float32)
    for e in range(len(counts)):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02), fmt=b_fmt)
    C = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), "f32", a_fmt=a_fmt, b_fmt=b_fmt)
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs, a_fmt=a_fmt, b_fmt=b_fmt)
    check(C.cpu().numpy().astype(np.float64), Cr, mass, "f32", f"grouped {a_fmt}x{b_fmt}")


def test_integer_e5m2_exact_in_fp32():
    """Integer-valued E5M2 values with power-of-two scales: exact FP32 output."""
    log("e5m2 integer exactness")
    tab = oracle.decode_table("e5m2")
    ints = np.array([c for c in range(256) if np.isfinite(tab[c]) and tab[c] == np.round(tab[c])
                     and abs(tab[c]) <= 16], np.uint8)
    rng = np.random.default_rng(5)
    M, N, K = 256, 392, 512
    A = ints[rng.integers(0, len(ints), (M, K))]
    B = ints[rng.integers(0, len(ints), (N, K))]
    sA = np.exp2(rng.integers(-3, 4, (2, 4))).astype(np.float32)
    sB = np.exp2(rng.integers(-3, 4, (4, 4))).astype(np.float32)
    C = dg.gemm_fp8_blockscaled(t(A), t(sA), t(B), t(sB), "f32", a_fmt="e5m2", b_fmt="e5m2")
    torch.cuda.synchronize()
    Cr, _ = oracle.gemm_blockscaled(A, sA, B, sB, a_fmt="e5m2", b_fmt="e5m2")
    assert np.abs(Cr).max() < 2 ** 24
    np.testing.assert_array_equal(C.cpu().numpy().astype(np.float64), Cr)


def test_e5m2_subnormal_operands():
    """Operands made mostly of E5M2 subnormal codes (exponent field 0): they
    reach the FP16 matrix cores as FP16 subnormals and must not be flushed."""
    log("e5m2 subnormals")
    rng = np.random.default_rng(6)
    M, N, K = 128, 256, 256
    sub = np.array([c for c in range(256) if (c >> 2) & 0x1F == 0], np.uint8)     # +-0 .. 3 * 2^-16
    normal = np.array([c for c in range(256) if 0 < (c >> 2) & 0x1F < 0x1F], np.uint8)
    A = sub[rng.integers(0, len(sub), (M, K))]
    B = np.where(rng.random((N, K)) < 0.5, sub[rng.integers(0, len(sub), (N, K))],
                 normal[rng.integers(0, len(normal), (N, K))]).astype(np.uint8)
    sA = np.full((1, 2), 2.0 ** 20, np.float32)
    sB = np.full((2, 2), 1.0, np.float32)
    C = dg.gemm_fp8_blockscaled(t(A), t(sA), t(B), t(sB), "f32", a_fmt="e5m2", b_fmt="e5m2")
    torch.cuda.synchronize()
    Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB, a_fmt="e5m2", b_fmt="e5m2")
    assert np.count_nonzero(Cr) > 0.9 * Cr.size
    check(C.cpu().numpy().astype(np.float64), Cr, mass, "f32", "e5m2 subnormals")


def test_full_size_e5m2_full():
    log("e5m2 4096^3 bf16, every output")
    p = I.dense_problem(4096, 4096, 4096, seed=2, out_dtype="bf16", block_log2_range=4.0,
                        a_fmt="e5m2", b_fmt="e5m2")
    Cg = run_dense(p)
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, a_fmt="e5m2", b_fmt="e5m2")
    check(Cg, Cr, mass, "bf16", "4096^3 e5m2")
