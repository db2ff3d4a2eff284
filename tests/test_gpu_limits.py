"""The largest K the library accepts (2^22, and 2^22 - 16 with a partial last
K-block) on the few-rows and the tiled kernels, against the CPU oracle.
Operands are random finite E4M3 codes with log-uniform block scales (no
quantisation pass: the matrices are large).  Needs a GPU."""
import sys

import numpy as np
import pytest
import torch

import parity_log

import oracle
from moe_grouped_gemm_block_amd import dg

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KMAX = 1 << 22


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()


def finite_codes(rng, shape):
    """Uniform over the 254 finite E4M3 codes, built in place as uint8 (the
    operands here are gigabytes)."""
    v = rng.integers(0, 254, shape, dtype=np.uint8)          # 0 .. 253
    np.add(v, v >= 0x7F, out=v, casting="unsafe")             # skip 0x7F; 0xFF is never reached
    return v


def operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    Kb = -(-K // 128)
    A = finite_codes(rng, (M, K))
    B = finite_codes(rng, (N, K))
    sA = np.exp2(rng.uniform(-8, 8, (-(-M // 128), Kb))).astype(np.float32)
    sB = np.exp2(rng.uniform(-8, 8, (-(-N // 128), Kb))).astype(np.float32)
    return A, sA, B, sB


def run(A, sA, B, sB, out):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    C = dg.gemm_fp8_blockscaled(t(A), t(sA), t(B), t(sB), out)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def check(Cg, Cr, mass, out, what):
    bound = oracle.tolerance(Cr, mass, out)
    err = np.abs(Cg - Cr)
    log(f"  {what}: max err/bound = {float((err / bound).max()):.3g}")
    parity_log.record(f"limits {what}", float((err / bound).max()))
    assert np.all(np.isfinite(Cg))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


@pytest.mark.parametrize("K", [KMAX, KMAX - 16])
def test_max_k_few_rows(K):
    log(f"limits: few rows 3 x 24 x {K}")
    A, sA, B, sB = operands(3, 24, K, seed=K % 97)
    Cg = run(A, sA, B, sB, "f32")
    Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    check(Cg, Cr, mass, "f32", f"3x24x{K}")


def test_max_k_tiled_sampled():
    K = KMAX - 16
    log(f"limits: tiled 130 x 520 x {K}, sampled")
    A, sA, B, sB = operands(130, 520, K, seed=5)
    Cg = run(A, sA, B, sB, "bf16")
    rows = np.array([0, 64, 127, 128, 129])
    cols = np.array([0, 255, 256, 511, 512, 519])
    Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB, rows=rows, cols=cols)
    check(Cg[np.ix_(rows, cols)], Cr, mass, "bf16", f"130x520x{K} sampled")
