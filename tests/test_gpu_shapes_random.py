"""Seeded random dense and grouped shapes through the automatic tile choice (the host picks
among seven tile shapes from M, N and the CU count, and may split a grid
into a main launch and a last-round launch; six dense cases are sized for the
shared-B 256 x 256 tile), each compared with the CPU
oracle to the parity bound.  Rows are sampled for the larger shapes, always
including the first and last rows of every 128-row tile.  Needs a GPU."""
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
    # dense shapes that take the shared-B 256 x 256 tile (M a multiple of 256,
    # whole rounds of 256 tiles on 256 CUs) with ragged N and random K
    for M, n_tiles in ((4096, 16), (2048, 32), (8192, 8), (1024, 64), (4096, 32), (512, 128)):
        N = 256 * n_tiles - int(rng.integers(0, 256))
        K = int(16 * rng.integers(1, 40))
        out.append((M, N, K, "bf16" if rng.random() < 0.5 else "f32"))
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
    parity_log.record(f"random {M}x{N}x{K} {out}", ratio)
    assert np.all(np.isfinite(Cg)) and ratio <= 1.0


def grouped_cases(n=10, seed=77):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        G = int(rng.integers(1, 12))
        counts = [int(c) if rng.random() > 0.2 else 0 for c in rng.integers(1, 700, G)]
        N = int(rng.choice([rng.integers(8, 600), rng.integers(600, 3000)]))
        K = int(16 * rng.integers(1, 24))
        out.append((tuple(counts), N, K, "bf16" if i % 2 else "f32"))
    return out


@pytest.mark.parametrize("counts,N,K,out", grouped_cases())
def test_random_grouped(counts, N, K, out):
    """Experts with random row counts (some empty), each segment padded to a
    multiple of 128 rows with zero rows; padding rows must come out zero."""
    rng = np.random.default_rng(sum(counts) + N + K)
    G = len(counts)
    offs = np.concatenate([[0], np.cumsum([-(-c // 128) * 128 for c in counts])]).astype(np.int32)
    A = np.zeros((int(offs[-1]), K), np.float32)
    for e, c in enumerate(counts):
        A[offs[e]:offs[e] + c] = rng.standard_normal((c, K), dtype=np.float32)
    qA, sA = I.quantize(A)
    Kb = -(-K // 128)
    qB = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, -(-N // 128), Kb), np.float32)
    for e in range(G):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    C = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), out)
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy().astype(np.float64)
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs)
    ratio = float((np.abs(Cg - Cr) / oracle.tolerance(Cr, mass, out)).max()) if Cg.size else 0.0
    log(f"  random grouped G={G} rows={int(offs[-1])} N={N} K={K} {out}: max err/bound = {ratio:.3g}")
    parity_log.record(f"random grouped G={G} N={N} K={K} {out}", ratio)
    assert np.all(np.isfinite(Cg)) and ratio <= 1.0
    for e, c in enumerate(counts):
        assert np.all(Cg[offs[e] + c:offs[e + 1]] == 0)
