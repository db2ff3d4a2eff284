"""Parity of the GEMMs with one A scale per row and 128-wide K-block (the
1 x 128 granularity, sa_rows = 1) through the C-ABI against the CPU oracle.
Needs a GPU.  Same bar as the 128 x 128 path: |C_gpu - C_ref| <= 1e-5 * mass
+ 1e-6 (FP32 out), plus 2^-8 |C_ref| for BF16 out."""
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
    log(f"  {what}: max err/bound = {float((err / bound).max()):.3g}")
    parity_log.record(f"rowscale {what}", float((err / bound).max()))
    assert np.all(np.isfinite(Cg))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


def run_dense(p, raw=False):
    if raw:      # straight through the C entry point, no shape inference
        C = torch.empty((p.M, p.N), dtype=torch.float32 if p.out_dtype == "f32" else torch.bfloat16,
                        device=DEV)
        A, sA, B, sB = t(p.A), t(p.sA), t(p.B), t(p.sB)
        st = dg.dg_gemm_fp8_ex(A.data_ptr(), dg.fmt_code(p.a_fmt), sA.data_ptr(), p.sa_rows, B.data_ptr(),
                               dg.fmt_code(p.b_fmt), sB.data_ptr(), C.data_ptr(), p.M, p.N, p.K,
                               dg.out_code(p.out_dtype), None)
        assert st == dg.DG_OK
    else:
        C = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), p.out_dtype, a_fmt=p.a_fmt,
                                    b_fmt=p.b_fmt)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def row_problem(M, N, K, seed, out="f32", a_fmt="e4m3", b_fmt="e4m3", spread=8.0, **kw):
    """Rows of A with magnitudes 2^U(-spread, spread) each, so a row read with
    another row's scale is far out of tolerance."""
    p = I.dense_problem(M, N, K, seed=seed, out_dtype=out, a_fmt=a_fmt, b_fmt=b_fmt, sa_rows=1, **kw)
    assert p.sA.shape == (M, K // 128)
    rng = np.random.default_rng(seed + 99)
    p.sA = (p.sA * np.exp2(rng.uniform(-spread, spread, (M, 1)))).astype(np.float32)
    return p


def oracle_of(p, rows=None):
    return oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, rows=rows, a_fmt=p.a_fmt, b_fmt=p.b_fmt, sa_rows=1)


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(65, 136, 128), (129, 264, 384), (300, 520, 256), (256, 128, 512),
                                   (200, 1032, 256)])
def test_dense_row_scales(M, N, K, out):
    log(f"rowscale dense {M}x{N}x{K} {out}")
    p = row_problem(M, N, K, seed=M + N + K, out=out)
    Cr, mass = oracle_of(p)
    check(run_dense(p), Cr, mass, out, f"{M}x{N}x{K} {out}")


@pytest.mark.parametrize("a_fmt,b_fmt", [("e5m2", "e5m2"), ("e4m3", "e5m2"), ("e5m2", "e4m3")])
@pytest.mark.parametrize("M,N,K", [(129, 264, 384), (40, 520, 256)])
def test_row_scales_with_e5m2(M, N, K, a_fmt, b_fmt):
    log(f"rowscale {a_fmt}x{b_fmt} {M}x{N}x{K}")
    p = row_problem(M, N, K, seed=M + N, out="bf16", a_fmt=a_fmt, b_fmt=b_fmt)
    Cr, mass = oracle_of(p)
    check(run_dense(p, raw=True), Cr, mass, "bf16", f"{a_fmt}x{b_fmt} {M}x{N}x{K}")


@pytest.mark.parametrize("M", [1, 5, 16, 17, 32, 33, 63, 64])
@pytest.mark.parametrize("N,K", [(520, 256), (12304, 384)])
def test_few_rows_row_scales(M, N, K):
    log(f"rowscale few rows {M}x{N}x{K}")
    p = row_problem(M, N, K, seed=M * 7 + N, out="bf16", b_std=0.02, outlier_frac=0.01)
    Cr, mass = oracle_of(p)
    check(run_dense(p, raw=True), Cr, mass, "bf16", f"few rows {M}x{N}x{K}")


def test_equal_row_scales_match_the_block_path():
    """Per-row scales equal within each 128-row block give the 128 x 128
    path's result (same arithmetic, so the outputs agree to the last bit)."""
    log("rowscale vs block path")
    p = I.dense_problem(300, 520, 384, seed=11, out_dtype="f32", block_log2_range=3.0)
    s1 = np.repeat(p.sA, 128, axis=0)[:300]
    Cb = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), "f32")
    Cr = dg.gemm_fp8_blockscaled(t(p.A), t(s1), t(p.B), t(p.sB), "f32")
    torch.cuda.synchronize()
    # different tiles (128x512 vs 128x256) still add the same K-block terms in the same order
    assert torch.equal(Cb, Cr)


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_grouped_row_scales(out):
    log(f"rowscale grouped {out}")
    rng = np.random.default_rng(3)
    counts, N, K = [300, 0, 130, 512, 1], 264, 384
    padded = [-(-c // 128) * 128 for c in counts]
    offs = np.concatenate([[0], np.cumsum(padded)]).astype(np.int32)
    A = np.zeros((int(offs[-1]), K), np.float32)
    for e, c in enumerate(counts):
        A[offs[e]:offs[e] + c] = (rng.standard_normal((c, K), dtype=np.float32)
                                  * np.exp2(rng.uniform(-6, 6, (c, 1))).astype(np.float32))
    qA, sA = I.quantize(A, rows=1)
    qB = np.empty((len(counts), N, K), np.uint8)
    sB = np.empty((len(counts), -(-N // 128), K // 128), np.float32)
    for e in range(len(counts)):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    C = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), out)
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs, sa_rows=1)
    check(C.float().cpu().numpy().astype(np.float64), Cr, mass, out, f"grouped {out}")


def test_gpu_quantised_tokens_feed_the_gemm():
    """Activations quantised on the GPU with 1 x 128 blocks go straight into
    the GEMM; the result matches the oracle GEMM on the oracle's own codes and
    per-token scales of the same activations (the codes are bit-exact, so
    the comparison is the GEMM's own tolerance)."""
    log("rowscale quantiser -> gemm")
    rng = np.random.default_rng(8)
    M, N, K = 200, 264, 512
    a = (rng.standard_normal((M, K)) * np.exp2(rng.uniform(-8, 8, (M, 1)))).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, sa = dg.quantize_fp8_blockscaled(torch.from_numpy(a).to(DEV), 1)
    qb, sb = dg.quantize_fp8_blockscaled(torch.from_numpy(b).to(DEV), 128)
    assert tuple(sa.shape) == (M, K // 128)
    C = dg.gemm_fp8_blockscaled(qa, sa, qb, sb, "f32")
    torch.cuda.synchronize()
    qao, sao = oracle.quantize_blockscaled(a, 1)
    qbo, sbo = oracle.quantize_blockscaled(b, 128)
    assert np.array_equal(qa.cpu().numpy(), qao) and np.array_equal(sa.cpu().numpy(), sao)
    Cr, mass = oracle.gemm_blockscaled(qao, sao, qbo, sbo, sa_rows=1)
    check(C.cpu().numpy().astype(np.float64), Cr, mass, "f32", "quantiser -> gemm")


def test_full_size_dense_row_scales_full():
    log("rowscale 4096^3 bf16, every output")
    p = I.make_config(2, sa_rows=1)
    Cg = run_dense(p)
    Cr, mass = oracle_of(p)
    check(Cg, Cr, mass, "bf16", "4096^3 row scales")


def test_full_size_few_rows_row_scales():
    log("rowscale 64x12288x4096 bf16")
    p = I.make_config(3, sa_rows=1)
    Cr, mass = oracle_of(p)
    check(run_dense(p), Cr, mass, "bf16", "64x12288x4096")


def test_full_size_grouped_row_scales_sampled():
    log("rowscale moe g8 sampled")
    p = I.make_config(4, sa_rows=1)
    C = dg.grouped_gemm_fp8(t(p.A), t(p.sA), t(p.B), t(p.sB), t(p.group_offsets), p.out_dtype)
    torch.cuda.synchronize()
    Cg = C.float().cpu().numpy().astype(np.float64)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.integers(0, p.M, 48), p.group_offsets[:-1], [p.M - 1]]))
    Cr, mass = oracle.grouped_gemm(p.A, p.sA, p.B, p.sB, p.group_offsets, rows=rows, sa_rows=1)
    check(Cg[rows], Cr, mass, "bf16", "moe g8 sampled")
