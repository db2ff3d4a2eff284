"""Seeded random shapes through the automatic tile choice (the host picks
among seven tile shapes from M, N and the CU count, and may split a grid
into a main launch and a last-round launch), each compared with the CPU
oracle to the parity bound.  Rows are sampled for the larger shapes, always
including the first and last rows of every 128-row tile.  Needs a GPU."""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_block_amd import dg
from moe_grouped_gemm_block_amd import inputs as I

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cases(n=24, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([rng.integers(65, 600), rng.integers(600, 4600)]))
        N = int(rng.choice([rng.integers(8, 700), rng.integers(700, 5000)]))
        K = int(16 * rng.integers(1, 40))
        out.append((M, N, K, "bf16" if i % 3 else "f32"))
    # grids around the tile-choice boundaries (one round of 128 x 512 tiles,
    # a last round of 1 .. 4 row tiles)
    out += [(2048, 4096, 256, "bf16"), (33 * 128, 2048, 128, "bf16"), (36 * 128 - 5, 1000, 144, "f32"),
            (1536, 4104, 128, "bf16")]
    return out


@pytest.mark.parametrize("M,N,K,out", cases())
def test_random_dense(M, N, K, out):
    p = I.dense_problem(M, N, K, seed=M * 7 + N * 3 + K, out_dtype=out, block_log2_range=3.0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    C = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), out)
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy().astype(np.float64)
    rows = None
    if M * N > 1 << 21:
        rng = np.random.default_rng(M + N)
        edges = [r for s in range(0, M, 128) for r in (s, s + 127) if r < M]
        rows = np.unique(np.concatenate([rng.choice(M, 48, replace=False), edges, [M - 1]]))
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, rows=rows)
    if rows is not None:
        Cg = Cg[rows]
    bound = oracle.tolerance(Cr, mass, out)
    ratio = float((np.abs(Cg - Cr) / bound).max())
    log(f"  random {M}x{N}x{K} {out}: max err/bound = {ratio:.3g}")
    assert np.all(np.isfinite(Cg)) and ratio <= 1.0
