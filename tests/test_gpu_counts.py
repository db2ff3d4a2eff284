"""Padding-aware grouped GEMM (dg_grouped_gemm_fp8_ex_counts) through the
C-ABI against the CPU oracle.

Each expert's padded segment carries a real row count; rows after it are
padding and must come out as exact zeros whatever A (and, with per-token
scales, sA) holds there -- here random codes including NaN codes.  Real rows
are compared with the oracle run on A with its padding rows zeroed, at the
parity bound.  Covered: a count of 0 on a non-empty segment (a tile of
padding only), counts at most 64 (a wave of padding rows computes nothing),
between 64 and 128, full segments, empty experts, split K, the 128 x 512
tiles with a narrow last round (workloads 4 and 5 in full), per-token A
scales, E5M2 B, and both output types.  With every count equal to its
segment length the result equals dg_grouped_gemm_fp8's bit for bit.
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


def padding_mask(offs, counts):
    pad = np.zeros(int(offs[-1]), bool)
    for e in range(len(counts)):
        pad[offs[e] + counts[e]:offs[e + 1]] = True
    return pad


def run_and_check(what, qA, sA, qB, sB, offs, counts, out, b_fmt="e4m3", sa_rows=128, garbage_seed=None):
    pad = padding_mask(offs, counts)
    A_dev, sA_dev = qA.copy(), sA.copy()
    if garbage_seed is not None:
        rng = np.random.default_rng(garbage_seed)
        A_dev[pad] = rng.integers(0, 256, size=(int(pad.sum()), qA.shape[1]), dtype=np.uint8)
        A_dev[pad, ::37] = 0x7F                 # NaN codes
        if sa_rows == 1:
            sA_dev[pad] = np.nan
    C = dg.grouped_gemm_fp8(t(A_dev), t(sA_dev), t(qB), t(sB), t(offs), out, b_fmt=b_fmt,
                            group_counts=t(np.asarray(counts, np.int32)))
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy().astype(np.float64)
    A_ref, sA_ref = qA.copy(), sA.copy()
    A_ref[pad] = 0
    if sa_rows == 1:
        sA_ref[pad] = 1.0
    Cr, mass = oracle.grouped_gemm(A_ref, sA_ref, qB, sB, offs, b_fmt=b_fmt, sa_rows=sa_rows)
    assert np.all(Cg[pad] == 0.0), "padding rows are not zero"
    real = ~pad
    bound = oracle.tolerance(Cr[real], mass[real], out)
    err = np.abs(Cg[real] - Cr[real])
    ratio = float((err / bound).max()) if real.any() else 0.0
    log(f"  counts {what}: max err/bound = {ratio:.3g} ({int(pad.sum())} padding rows zero)")
    parity_log.record(f"counts {what}", ratio)
    assert np.all(np.isfinite(Cg))
    assert ratio <= 1.0


def small_problem(counts, seg, N, K, seed, sa_rows=128, b_fmt="e4m3"):
    rng = np.random.default_rng(seed)
    offs = np.concatenate([[0], np.cumsum(seg)]).astype(np.int32)
    A = np.zeros((int(offs[-1]), K), np.float32)
    for e, c in enumerate(counts):
        A[offs[e]:offs[e] + c] = rng.standard_normal((c, K), dtype=np.float32)
    qA, sA = I.quantize(A, rows=sa_rows)
    G = len(counts)
    qB = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, -(-N // 128), -(-K // 128)), np.float32)
    for e in range(G):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02), fmt=b_fmt)
    return qA, sA, qB, sB, offs


# counts and padded segment lengths: a count of 0 on a 128-row segment (a
# tile of padding only), counts <= 64, between 64 and 128, full, empty
COUNTS = [200, 0, 60, 100, 128, 5, 0]
SEGS = [256, 0, 128, 128, 128, 128, 128]


@pytest.mark.parametrize("N,K,out,sa_rows,b_fmt", [
    (2048, 2048, "f32", 128, "e4m3"),          # 7 row tiles: K split 2 ways
    (1000, 640, "bf16", 128, "e4m3"),          # narrow tiles, ragged N, partial K-block
    (2048, 1024, "f32", 1, "e4m3"),            # per-token scales (NaN scales in the padding)
    (520, 256, "bf16", 128, "e5m2"),
])
def test_counts_small(N, K, out, sa_rows, b_fmt):
    log(f"counts small N={N} K={K} {out} sa_rows={sa_rows} {b_fmt}")
    qA, sA, qB, sB, offs = small_problem(COUNTS, SEGS, N, K, seed=N + K, sa_rows=sa_rows, b_fmt=b_fmt)
    run_and_check(f"small N={N} K={K} {out} sa_rows={sa_rows} {b_fmt}", qA, sA, qB, sB, offs, COUNTS, out,
                  b_fmt=b_fmt, sa_rows=sa_rows, garbage_seed=K)


@pytest.mark.parametrize("i", [4, 5])
def test_counts_workload(i):
    """Workloads 4 and 5 with their real per-expert counts, garbage in the
    padding rows, every output compared."""
    p = I.make_config(i)
    log(f"counts workload {i}: {p.name}")
    run_and_check(f"workload {i}", p.A, p.sA, p.B, p.sB, p.group_offsets, p.group_counts, p.out_dtype,
                  garbage_seed=i)


def test_full_counts_equal_plain_call():
    qA, sA, qB, sB, offs = small_problem([256, 100, 0, 300], [256, 128, 0, 384], 1024, 1024, seed=2)
    counts = np.diff(offs).astype(np.int32)
    C1 = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), "bf16", group_counts=t(counts))
    C2 = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), "bf16")
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
