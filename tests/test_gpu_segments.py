"""Parity of the grouped GEMM over packed (unpadded) expert segments with
per-row A scales -- the decode-time MoE layout -- through the C-ABI against
the CPU oracle.  Needs a GPU.  Bar: |C_gpu - C_ref| <= 1e-5 * mass + 1e-6
(FP32 out), plus 2^-8 |C_ref| for BF16 out."""
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


def check(Cg, Cr, mass, out_dtype, what):
    bound = oracle.tolerance(Cr, mass, out_dtype)
    err = np.abs(Cg - Cr)
    log(f"  {what}: max err/bound = {float((err / bound).max()) if err.size else 0:.3g}")
    parity_log.record(f"segments {what}", float((err / bound).max()) if err.size else 0.0)
    assert np.all(np.isfinite(Cg))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


def packed(counts, N, K, seed, a_fmt="e4m3", b_fmt="e4m3"):
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    M = int(offs[-1])
    A = (rng.standard_normal((M, K)) * np.exp2(rng.uniform(-6, 6, (M, 1)))).astype(np.float32)
    qA, sA = I.quantize(A, fmt=a_fmt, rows=1)
    G = len(counts)
    qB = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, -(-N // 128), K // 128), np.float32)
    for e in range(G):
        Be = rng.standard_normal((N, K)).astype(np.float32) * np.float32(0.02)
        Be *= np.exp2(rng.uniform(-3, 3)).astype(np.float32)
        qB[e], sB[e] = I.quantize(Be, fmt=b_fmt)
    return qA, sA, qB, sB, offs


def run(qA, sA, qB, sB, offs, out, a_fmt="e4m3", b_fmt="e4m3"):
    C = dg.grouped_gemm_fp8_segments(t(qA), t(sA), t(qB), t(sB), t(offs), out, a_fmt=a_fmt, b_fmt=b_fmt)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


CASES = [
    ([3, 0, 17, 64, 1], 264, 384),          # every chunk height, an empty expert
    ([16, 32, 33, 15, 0, 0, 2], 136, 256),  # chunk-height edges
    ([130, 0, 65, 7], 520, 256),            # segments longer than 64 rows: several chunks
    ([0, 0, 0, 5], 1032, 128),              # one K-block, leading empty experts
    ([1] * 40, 264, 512),                   # many one-row experts: wide slabs
]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("counts,N,K", CASES)
def test_segments(counts, N, K, out):
    log(f"segments {counts} N={N} K={K} {out}")
    qA, sA, qB, sB, offs = packed(counts, N, K, seed=sum(counts) + N)
    Cg = run(qA, sA, qB, sB, offs, out)
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs, sa_rows=1)
    check(Cg, Cr, mass, out, f"{counts} {out}")


@pytest.mark.parametrize("a_fmt,b_fmt", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
def test_segments_e5m2(a_fmt, b_fmt):
    log(f"segments {a_fmt}x{b_fmt}")
    counts, N, K = [5, 0, 40, 70], 264, 384
    qA, sA, qB, sB, offs = packed(counts, N, K, seed=7, a_fmt=a_fmt, b_fmt=b_fmt)
    Cg = run(qA, sA, qB, sB, offs, "bf16", a_fmt, b_fmt)
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs, sa_rows=1, a_fmt=a_fmt, b_fmt=b_fmt)
    check(Cg, Cr, mass, "bf16", f"{a_fmt}x{b_fmt}")


def test_one_expert_equals_the_dense_few_rows_path():
    """G = 1 with at most 64 rows runs the same few-rows arithmetic as the
    dense call with per-row scales, so the outputs agree to the last bit."""
    log("segments G=1 vs dense")
    qA, sA, qB, sB, offs = packed([45], 520, 384, seed=3)
    Cs = run(qA, sA, qB, sB, offs, "f32")
    Cd = dg.gemm_fp8_blockscaled(t(qA), t(sA), t(qB[0]), t(sB[0]), "f32")
    torch.cuda.synchronize()
    Cd = Cd.cpu().numpy().astype(np.float64)
    assert np.array_equal(Cs, Cd)


def test_empty_experts_leave_no_trace_and_repeat_bitwise():
    log("segments repeatability")
    qA, sA, qB, sB, offs = packed([0, 9, 0, 0, 60, 0], 264, 256, seed=4)
    C1 = run(qA, sA, qB, sB, offs, "bf16")
    C2 = run(qA, sA, qB, sB, offs, "bf16")
    assert np.array_equal(C1, C2)


def test_inconsistent_offsets_stay_in_bounds():
    """Offsets past M_total or decreasing are clamped by the kernel: rows
    outside [0, M_total) are never touched and the covered rows are right."""
    log("segments clamped offsets")
    qA, sA, qB, sB, _ = packed([10, 0, 6], 136, 256, seed=5)
    M = qA.shape[0]
    bad = np.array([0, 10, 4, 1000], np.int32)     # expert 1: [10, 4) -> empty; expert 2: [4, 16)
    guard = torch.full((M + 2, 136), 7.0, dtype=torch.float32, device=DEV)
    C = guard[1:M + 1]
    dg.grouped_gemm_fp8_segments(t(qA), t(sA), t(qB), t(sB), t(bad), "f32", C=C)
    torch.cuda.synchronize()
    g = guard.cpu().numpy()
    assert np.all(g[0] == 7.0) and np.all(g[M + 1] == 7.0)
    Cr, mass = oracle.gemm_blockscaled(qA[:10], sA[:10], qB[0], sB[0], sa_rows=1)
    Cg = C.cpu().numpy().astype(np.float64)
    # rows [4, 10) are written by expert 0 and expert 2 (a race by construction);
    # rows [0, 4) only by expert 0 and rows [10, 16) only by expert 2
    check(Cg[:4], Cr[:4], mass[:4], "f32", "expert 0 rows")
    Cr2, mass2 = oracle.gemm_blockscaled(qA[4:16], sA[4:16], qB[2], sB[2], sa_rows=1)
    check(Cg[10:16], Cr2[6:], mass2[6:], "f32", "expert 2 rows")


def test_decode_workload_full():
    log("segments decode workload (G=64, 128 tokens)")
    p = I.make_config(6)
    Cg = run(p.A, p.sA, p.B, p.sB, p.group_offsets, p.out_dtype)
    Cr, mass = oracle.grouped_gemm(p.A, p.sA, p.B, p.sB, p.group_offsets, sa_rows=1)
    check(Cg, Cr, mass, p.out_dtype, "decode workload")
