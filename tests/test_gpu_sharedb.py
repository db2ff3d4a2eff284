"""Parity of the shared-B 256 x 256 tile (csrc/gemm_sharedb.hpp) through the
C-ABI against the CPU oracle.  The library picks it for dense problems whose
256 x 256 tiles fill whole rounds of the 256 CUs; every shape below has 256
such tiles, so these calls go through the default dispatch.  Covered: a
partial last K-block, N tails with and without 16-byte aligned rows of C,
both output types, per-row A scales, E5M2 and mixed operand formats, and
the integer case that must be exact.  Every output is compared.  Needs a
GPU (the MI355X's 256 CUs: on another CU count the dispatch differs)."""
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run(p):
    C = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), p.out_dtype, a_fmt=p.a_fmt, b_fmt=p.b_fmt)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def check(p, what):
    Cg = run(p)
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, a_fmt=p.a_fmt, b_fmt=p.b_fmt, sa_rows=p.sa_rows)
    bound = oracle.tolerance(Cr, mass, p.out_dtype)
    err = np.abs(Cg - Cr)
    ratio = float((err / bound).max())
    log(f"  shared-B {what}: max err/bound = {ratio:.3g}")
    parity_log.record(f"shared-B {what}", ratio)
    assert np.all(np.isfinite(Cg))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


# M, N, K, out: 16 x 16 and 8 x 32 tiles of 256 x 256; K = 272 and 400 end in
# a partial K-block, K = 16 and 112 are one partial K-block, K = 128 one full
# one; N = 4080 (last tile 240 columns, rows of C 16-byte aligned) and
# N = 4090 (element-wise stores)
SHAPES = [(4096, 4096, 128, "f32"), (4096, 4096, 272, "bf16"), (4096, 4080, 384, "f32"),
          (4096, 4090, 256, "f32"), (4096, 4090, 144, "bf16"), (2048, 8192, 400, "f32"),
          (4096, 4096, 16, "f32"), (4096, 4096, 112, "bf16")]


@pytest.mark.parametrize("M,N,K,out", SHAPES)
def test_sharedb_shapes(M, N, K, out):
    log(f"shared-B {M}x{N}x{K} {out}")
    p = I.dense_problem(M, N, K, seed=M + N + K, out_dtype=out, block_log2_range=4.0)
    check(p, f"{M}x{N}x{K} {out}")


@pytest.mark.parametrize("a_fmt,b_fmt", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_sharedb_formats(a_fmt, b_fmt):
    M = N = 4096
    K = 256
    log(f"shared-B formats {a_fmt} x {b_fmt}")
    p = I.dense_problem(M, N, K, seed=7, out_dtype="f32", block_log2_range=3.0, a_fmt=a_fmt, b_fmt=b_fmt)
    check(p, f"{a_fmt}x{b_fmt} {M}x{N}x{K} f32")


@pytest.mark.parametrize("out,K", [("f32", 400), ("bf16", 400), ("f32", 112), ("bf16", 640)])
def test_sharedb_row_scales(out, K):
    M = N = 4096
    log(f"shared-B per-row A scales {out} K={K}")
    p = I.dense_problem(M, N, K, seed=11, out_dtype=out, block_log2_range=3.0, sa_rows=1)
    check(p, f"1x128 A scales {M}x{N}x{K} {out}")


def test_sharedb_integer_exact():
    """Integer E4M3 values with power-of-two scales: FP32 output is exact."""
    rng = np.random.default_rng(3)
    M = N = 4096
    K = 256
    vals = np.arange(-8, 9).astype(np.float32)
    code = lambda x: torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    A = code(rng.choice(vals, size=(M, K)).astype(np.float32))
    B = code(rng.choice(vals, size=(N, K)).astype(np.float32))
    sA = np.exp2(rng.integers(-3, 4, size=(M // 128, K // 128))).astype(np.float32)
    sB = np.exp2(rng.integers(-3, 4, size=(N // 128, K // 128))).astype(np.float32)
    p = I.Problem("int", A, sA, B, sB, M, N, K, "f32", 0)
    Cg = run(p)
    Cr, _ = oracle.gemm_blockscaled(A, sA, B, sB)
    assert np.abs(Cr).max() < 2 ** 24
    np.testing.assert_array_equal(Cg, Cr)
