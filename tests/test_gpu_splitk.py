"""Parity of the split-K path through the C-ABI against the CPU oracle.

Grids with at most half as many workgroups as CUs run with K split over
several copies of the tile grid: every copy sums its own range of K-blocks
(each with its own rescale), stores an FP32 partial tile into a workspace,
and a second kernel adds the copies in a fixed order.  Every shape below is
small enough for the automatic plan to split it (on the MI355X's 256 CUs):
ragged rows and columns, a partial last K-block, more splits than fit
evenly into the K-blocks, both output types, per-row A scales, E5M2 and
mixed formats, and a grouped problem.
Every output is compared; the split result is also bitwise repeatable.
Needs a GPU."""
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


def host(C):
    return C.float().cpu().numpy().astype(np.float64)


def check(what, Cg, Cr, mass, out):
    bound = oracle.tolerance(Cr, mass, out)
    err = np.abs(Cg - Cr)
    ratio = float((err / bound).max())
    log(f"  split-K {what}: max err/bound = {ratio:.3g}")
    parity_log.record(f"split-K {what}", ratio)
    assert np.all(np.isfinite(Cg))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


# M, N, K, out, A-scale rows.  The automatic plan splits K on the 128 x 128
# tile into S = min(CUs / tiles, K-blocks / 8, 8) parts; here S = 4, 2
# (17 K-blocks, the last partial: 8 + 9), 3 (25 K-blocks: 8 + 8 + 9, ragged
# rows and columns, FP32 partial rows padded to 4), 2, 4, 2 and 8.
SHAPES = [(256, 4096, 4096, "bf16", 128), (128, 4096, 2064, "f32", 128), (200, 4090, 3200, "f32", 128),
          (136, 1000, 2048, "bf16", 128), (128, 2048, 4096, "f32", 128), (256, 3000, 2048, "f32", 1),
          (130, 2048, 8192, "bf16", 1)]


@pytest.mark.parametrize("M,N,K,out,sa_rows", SHAPES)
def test_splitk_dense(M, N, K, out, sa_rows):
    log(f"split-K dense {M}x{N}x{K} {out} sa_rows={sa_rows}")
    p = I.dense_problem(M, N, K, seed=M * 7 + N + K, out_dtype=out, block_log2_range=3.0, sa_rows=sa_rows)
    args = (t(p.A), t(p.sA), t(p.B), t(p.sB), out)
    C1 = dg.gemm_fp8_blockscaled(*args)
    C2 = dg.gemm_fp8_blockscaled(*args)
    torch.cuda.synchronize()
    assert torch.equal(C1, C2), "split-K result not repeatable"
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, sa_rows=sa_rows)
    check(f"{M}x{N}x{K} {out} sa_rows={sa_rows}", host(C1), Cr, mass, out)


@pytest.mark.parametrize("a_fmt,b_fmt", [("e5m2", "e5m2"), ("e4m3", "e5m2")])
def test_splitk_formats(a_fmt, b_fmt):
    M, N, K = 256, 2048, 2048
    log(f"split-K formats {a_fmt} x {b_fmt}")
    p = I.dense_problem(M, N, K, seed=5, out_dtype="f32", block_log2_range=3.0, a_fmt=a_fmt, b_fmt=b_fmt)
    C = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), "f32", a_fmt=a_fmt, b_fmt=b_fmt)
    torch.cuda.synchronize()
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, a_fmt=a_fmt, b_fmt=b_fmt)
    check(f"{a_fmt}x{b_fmt} {M}x{N}x{K} f32", host(C), Cr, mass, "f32")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_splitk_grouped(out):
    """A small MoE problem (4 experts, one empty, 4 row tiles in all): the
    whole grid is split 2 ways."""
    rng = np.random.default_rng(11)
    counts, N, K = [200, 0, 60, 100], 2048, 2048
    offs = np.concatenate([[0], np.cumsum([-(-c // 128) * 128 for c in counts])]).astype(np.int32)
    A = np.zeros((int(offs[-1]), K), np.float32)
    for e, c in enumerate(counts):
        A[offs[e]:offs[e] + c] = rng.standard_normal((c, K), dtype=np.float32)
    qA, sA = I.quantize(A)
    qB = np.empty((4, N, K), np.uint8)
    sB = np.empty((4, -(-N // 128), K // 128), np.float32)
    for e in range(4):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    log(f"split-K grouped {out}")
    C = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), out)
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs)
    check(f"grouped 4 experts N={N} K={K} {out}", host(C), Cr, mass, out)


def random_split_shapes(n=8, seed=17):
    """Seeded shapes the automatic plan splits: 1-4 row tiles (M > 64, so
    not the few-rows kernel), N up to 3000, K from 2048 to 8192 in steps of
    16 (K-blocks >= 16, the last one often partial); each (S = min(CUs /
    128-by-128 tiles, K-blocks / 8, 8)) >= 2 on 256 CUs."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(65, 513))
        N = int(rng.integers(16, 3001))
        K = int(rng.integers(128, 513)) * 16
        tiles = -(-M // 128) * -(-N // 128)
        S = min(256 // tiles, (-(-K // 128)) // 8, 8)
        if S >= 2:
            out.append((M, N, K, "f32" if len(out) % 2 else "bf16", S))
    return out


@pytest.mark.parametrize("M,N,K,out,S", random_split_shapes())
def test_splitk_random(M, N, K, out, S):
    log(f"split-K random {M}x{N}x{K} {out} (S={S})")
    p = I.dense_problem(M, N, K, seed=M + N + K, out_dtype=out, block_log2_range=3.0)
    C = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), out)
    torch.cuda.synchronize()
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB)
    check(f"random {M}x{N}x{K} {out} S={S}", host(C), Cr, mass, out)



def test_splitk_concurrent_streams():
    """Split-K calls on three streams at once, four rounds without a
    synchronisation in between.  Each stream has its own workspace, so every
    result equals the same call run alone bit for bit, and the oracle within
    the bound."""
    shapes = [(256, 4096, 4096, "bf16"), (128, 2048, 4096, "f32"), (136, 1000, 2048, "bf16")]
    probs = [I.dense_problem(M, N, K, seed=40 + i, out_dtype=out, block_log2_range=3.0)
             for i, (M, N, K, out) in enumerate(shapes)]
    dev = [(t(p.A), t(p.sA), t(p.B), t(p.sB)) for p in probs]
    alone = []
    for p, d in zip(probs, dev):
        C = dg.gemm_fp8_blockscaled(*d, p.out_dtype)
        torch.cuda.synchronize()
        alone.append(host(C))
    streams = [torch.cuda.Stream() for _ in probs]
    outs = [[] for _ in probs]
    torch.cuda.synchronize()
    for _ in range(4):
        for i, (p, d, s) in enumerate(zip(probs, dev, streams)):
            with torch.cuda.stream(s):
                outs[i].append(dg.gemm_fp8_blockscaled(*d, p.out_dtype, stream=s))
    torch.cuda.synchronize()
    for i, p in enumerate(probs):
        log(f"split-K stream {i}: {p.M}x{p.N}x{p.K} {p.out_dtype}")
        for C in outs[i]:
            assert np.array_equal(host(C), alone[i]), f"stream {i}: result differs from the call alone"
        Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB)
        check(f"stream {i} {p.M}x{p.N}x{p.K}", alone[i], Cr, mass, p.out_dtype)
