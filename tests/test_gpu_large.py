"""Row counts whose byte offsets in A pass 2^32: M = 2^20 rows at K = 4096
(4 GiB of A) through the dense 256 x 256 path, the 128-row tiled path
(M = 2^20 + 128) and the grouped path (four experts over the 2^20 rows),
compared with the CPU oracle on sampled rows spread over the whole range.
Operands are random finite E4M3 codes with log-uniform block scales, generated
in chunks straight into device memory (only the sampled rows stay on the
host).  Needs a GPU."""
import sys

import numpy as np
import pytest
import torch

import parity_log

import oracle
from moe_grouped_gemm_block_amd import dg

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
M_BIG = 1 << 20
N, K = 256, 4096
KB = K // 128
CHUNK = 1 << 14                                  # rows per generated chunk (64 MiB)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def finite_codes(rng, shape):
    """Uniform over the 254 finite E4M3 codes (0x7F and 0xFF skipped)."""
    v = rng.integers(0, 254, shape, dtype=np.uint8)
    np.add(v, v >= 0x7F, out=v, casting="unsafe")
    return v


SAMPLE = np.array(sorted({0, 1, 127, 128, 255, 256, (1 << 19) - 1, 1 << 19, (1 << 19) + 128,
                          M_BIG - 257, M_BIG - 129, M_BIG - 128, M_BIG - 1, M_BIG, M_BIG + 127}
                         | set(np.random.default_rng(9).integers(0, M_BIG + 128, 17).tolist())))


@pytest.fixture(scope="module")
def big():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()
    rows = M_BIG + 128
    rng = np.random.default_rng(2026)
    A = torch.empty((rows, K), dtype=torch.uint8, device=DEV)
    sampled = {}
    for r0 in range(0, rows, CHUNK):
        r1 = min(rows, r0 + CHUNK)
        part = finite_codes(rng, (r1 - r0, K))
        A[r0:r1].copy_(torch.from_numpy(part))
        for r in SAMPLE[(SAMPLE >= r0) & (SAMPLE < r1)]:
            sampled[int(r)] = part[r - r0].copy()
    torch.cuda.synchronize()
    sA = np.exp2(rng.uniform(-6, 6, (rows // 128, KB))).astype(np.float32)
    B = finite_codes(rng, (4, N, K))
    sB = np.exp2(rng.uniform(-6, 6, (4, N // 128, KB))).astype(np.float32)
    log(f"large operands: A {rows} x {K} on the device, {len(sampled)} rows sampled")
    yield A, sampled, sA, B, sB
    del A
    torch.cuda.empty_cache()


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def reference_rows(rows, sampled, sA, B, sB):
    """Oracle rows: each sampled row with its own 128-row block's scales."""
    Cr, mass = [], []
    for r in rows:
        c, m = oracle.gemm_blockscaled(sampled[int(r)][None, :], sA[int(r) // 128][None, :], B, sB)
        Cr.append(c[0])
        mass.append(m[0])
    return np.array(Cr), np.array(mass)


def check(Cg_rows, Cr, mass, out, what):
    bound = oracle.tolerance(Cr, mass, out)
    err = np.abs(Cg_rows - Cr)
    ratio = float((err / bound).max())
    log(f"  {what}: max err/bound = {ratio:.3g}")
    parity_log.record(f"large {what}", ratio)
    assert np.all(np.isfinite(Cg_rows))
    bad = np.argwhere(err > bound)
    assert len(bad) == 0, f"{len(bad)} elements out of tolerance, first {bad[:5].tolist()}"


@pytest.mark.parametrize("M,out", [(M_BIG, "bf16"), (M_BIG + 128, "f32")],
                         ids=["dense_256x256_tile", "tiled_128_rows"])
def test_large_m_dense(big, M, out):
    A, sampled, sA, B, sB = big
    log(f"large dense {M}x{N}x{K} {out}")
    C = dg.gemm_fp8_blockscaled(A[:M], t(sA[:M // 128]), t(B[0]), t(sB[0]), out)
    torch.cuda.synchronize()
    rows = SAMPLE[SAMPLE < M]
    Cg = C[t(rows).long()].float().cpu().numpy().astype(np.float64)
    del C
    Cr, mass = reference_rows(rows, sampled, sA, B[0], sB[0])
    check(Cg, Cr, mass, out, f"{M}x{N}x{K} {out}")


def test_large_m_grouped(big):
    A, sampled, sA, B, sB = big
    offs = np.array([0, 1 << 18, (1 << 19) + 3 * 128, M_BIG - 5 * 128, M_BIG], np.int32)
    log(f"large grouped {M_BIG}x{N}x{K}, offsets {offs.tolist()}")
    C = dg.grouped_gemm_fp8(A[:M_BIG], t(sA[:M_BIG // 128]), t(B), t(sB), t(offs), "bf16")
    torch.cuda.synchronize()
    rows = SAMPLE[SAMPLE < M_BIG]
    Cg = C[t(rows).long()].float().cpu().numpy().astype(np.float64)
    del C
    Cr, mass = [], []
    for r in rows:
        e = int(np.searchsorted(offs, r, side="right")) - 1
        c, m = reference_rows([r], sampled, sA, B[e], sB[e])
        Cr.append(c[0])
        mass.append(m[0])
    check(Cg, np.array(Cr), np.array(mass), "bf16", f"grouped {M_BIG}x{N}x{K}")
