"""Parity of every GEMM entry point with K and N tails (K a multiple of 16
but not of 128, so the last K-block is partial with its own scales; N not a
multiple of 8, so rows of C are not 16-byte aligned) against the CPU oracle,
through the C-ABI.  Needs a GPU.  Bar: |C_gpu - C_ref| <= 1e-5 * mass + 1e-6
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
    parity_log.record(f"tails {what}", float((err / bound).max()) if err.size else 0.0)
    assert np.all(np.isfinite(Cg))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


def guarded_dense(p, sa_rows=128):
    """Run through the C entry point into a buffer with guard elements on both
    sides of C; return C and whether the guards are intact."""
    dt = torch.float32 if p.out_dtype == "f32" else torch.bfloat16
    G = 64
    buf = torch.full((p.M * p.N + 2 * G,), 3.0, dtype=dt, device=DEV)
    # C must be 16-byte aligned: the guard is 64 elements (128 or 256 bytes)
    C = buf[G:G + p.M * p.N]
    A, sA, B, sB = t(p.A), t(p.sA), t(p.B), t(p.sB)
    st = dg.dg_gemm_fp8_ex(A.data_ptr(), dg.fmt_code(p.a_fmt), sA.data_ptr(), sa_rows, B.data_ptr(),
                           dg.fmt_code(p.b_fmt), sB.data_ptr(), C.data_ptr(), p.M, p.N, p.K,
                           dg.out_code(p.out_dtype), None)
    assert st == dg.DG_OK, dg.dg_status_string(st)
    torch.cuda.synchronize()
    b = buf.float().cpu().numpy()
    intact = bool(np.all(b[:G] == 3.0) and np.all(b[G + p.M * p.N:] == 3.0))
    return C.float().cpu().numpy().astype(np.float64).reshape(p.M, p.N), intact


DENSE = [(130, 13, 144), (200, 519, 400), (129, 1, 16), (257, 263, 272), (300, 1000, 4112), (65, 7, 112),
         (1, 13, 144), (17, 519, 400), (33, 100, 48), (64, 12301, 528)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", DENSE)
def test_dense_tails(M, N, K, out):
    log(f"tails dense {M}x{N}x{K} {out}")
    p = I.dense_problem(M, N, K, seed=M + N + K, out_dtype=out, block_log2_range=3.0)
    assert p.sA.shape[1] == -(-K // 128)
    Cg, intact = guarded_dense(p)
    assert intact, "write outside C"
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB)
    check(Cg, Cr, mass, out, f"{M}x{N}x{K} {out}")


def test_wide_tile_with_tails_sampled():
    """Enough tiles for the 128 x 512 tile, N not a multiple of 8, a 16-column K tail."""
    log("tails 128x512 tile 2048x4100x1040")
    p = I.dense_problem(2048, 4100, 1040, seed=9, out_dtype="bf16", block_log2_range=3.0)
    Cg, intact = guarded_dense(p)
    assert intact
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.integers(0, 2048, 24), [0, 127, 128, 2047]]))
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, rows=rows)
    check(Cg[rows], Cr, mass, "bf16", "2048x4100x1040 sampled rows")


@pytest.mark.parametrize("M,N,K", [(130, 263, 272), (40, 100, 176), (300, 129, 16)])
def test_row_scales_with_tails(M, N, K):
    log(f"tails row scales {M}x{N}x{K}")
    p = I.dense_problem(M, N, K, seed=M + K, out_dtype="bf16", sa_rows=1)
    Cg, intact = guarded_dense(p, sa_rows=1)
    assert intact
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, sa_rows=1)
    check(Cg, Cr, mass, "bf16", f"row scales {M}x{N}x{K}")


@pytest.mark.parametrize("a_fmt,b_fmt,M,N,K", [("e5m2", "e5m2", 129, 136, 144), ("e4m3", "e5m2", 20, 77, 48),
                                               ("e5m2", "e4m3", 200, 9, 400)])
def test_e5m2_with_tails(a_fmt, b_fmt, M, N, K):
    log(f"tails {a_fmt}x{b_fmt} {M}x{N}x{K}")
    p = I.dense_problem(M, N, K, seed=N + K, out_dtype="f32", a_fmt=a_fmt, b_fmt=b_fmt)
    Cg, intact = guarded_dense(p)
    assert intact
    Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, a_fmt=a_fmt, b_fmt=b_fmt)
    check(Cg, Cr, mass, "f32", f"{a_fmt}x{b_fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_grouped_tails(out):
    log(f"tails grouped {out}")
    rng = np.random.default_rng(5)
    counts, N, K = [300, 0, 130], 263, 272
    padded = [-(-c // 128) * 128 for c in counts]
    offs = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    A = np.zeros((int(offs[-1]), K), np.float32)
    for e, c in enumerate(counts):
        A[offs[e]:offs[e] + c] = rng.standard_normal((c, K), dtype=np.float32)
    qA, sA = I.quantize(A)
    qB = np.empty((3, N, K), np.uint8)
    sB = np.empty((3, 3, 3), np.float32)
    for e in range(3):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    C = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), out)
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs)
    check(C.float().cpu().numpy().astype(np.float64), Cr, mass, out, f"grouped {out}")


def test_segments_tails():
    log("tails packed segments")
    rng = np.random.default_rng(6)
    counts, N, K = [3, 0, 40, 70], 101, 208
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qA, sA = I.quantize(rng.standard_normal((int(offs[-1]), K)).astype(np.float32), rows=1)
    qB = np.empty((4, N, K), np.uint8)
    sB = np.empty((4, 1, 2), np.float32)
    for e in range(4):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    C = dg.grouped_gemm_fp8_segments(t(qA), t(sA), t(qB), t(sB), t(offs), "bf16")
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs, sa_rows=1)
    check(C.float().cpu().numpy().astype(np.float64), Cr, mass, "bf16", "segments")


def test_k_tail_equals_zero_padded_k():
    """The kernel on K = 144 and on the same operands zero-padded to K = 256
    (same scales) give the same bits: the tail reads exact zeros."""
    log("tails: K=144 vs zero-padded K=256")
    p = I.dense_problem(260, 520, 144, seed=4, out_dtype="f32")
    Ap = np.zeros((260, 256), np.uint8)
    Bp = np.zeros((520, 256), np.uint8)
    Ap[:, :144], Bp[:, :144] = p.A, p.B
    C1 = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), "f32")
    C2 = dg.gemm_fp8_blockscaled(t(Ap), t(p.sA), t(Bp), t(p.sB), "f32")
    torch.cuda.synchronize()
    assert torch.equal(C1, C2)
