"""Child process of tests/test_gpu_overrides.py (not collected by pytest).

The library reads DG_FORCE_TILE, DG_TAIL_TILE and DG_SPLITK once per process, so each
setting is checked in a process of its own: a few dense and grouped GEMMs
through the C-ABI against the CPU oracle, with the same tolerance as the
parity tests.  Exit status 0 when every case is inside it."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from moe_grouped_gemm_block_amd import dg  # noqa: E402
from moe_grouped_gemm_block_amd import inputs as I  # noqa: E402

DEV = "cuda:0"


def t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def ratio(Cg, Cr, mass, out):
    return float((np.abs(Cg - Cr) / oracle.tolerance(Cr, mass, out)).max())


def main():
    setting = {k: os.environ.get(k) for k in ("DG_FORCE_TILE", "DG_TAIL_TILE", "DG_SPLITK")}
    print(f"override child {setting}", flush=True)
    worst = 0.0
    # dense: ragged, and a grid with a partial last round of 128 x 512 tiles
    for (M, N, K, sampled) in [(300, 1032, 384, False), (33 * 128, 1024, 256, True)]:
        p = I.dense_problem(M, N, K, seed=M + N, out_dtype="bf16", block_log2_range=3.0)
        C = dg.gemm_fp8_blockscaled(t(p.A), t(p.sA), t(p.B), t(p.sB), "bf16")
        torch.cuda.synchronize()
        Cg = C.float().cpu().numpy().astype(np.float64)
        rows = (np.unique(np.concatenate([np.arange(0, M, 97), [127, 128, 32 * 128 - 1, 32 * 128, M - 1]]))
                if sampled else None)
        rows = rows[rows < M] if rows is not None else None
        Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB, rows=rows)
        r = ratio(Cg if rows is None else Cg[rows], Cr, mass, "bf16")
        print(f"  dense {M}x{N}x{K}: max err/bound = {r:.3g}", flush=True)
        worst = max(worst, r)
    # grouped with an empty expert, FP32 out
    rng = np.random.default_rng(1)
    counts, N, K = [300, 0, 130, 512], 520, 256
    offs = np.concatenate([[0], np.cumsum([-(-c // 128) * 128 for c in counts])]).astype(np.int32)
    A = np.zeros((int(offs[-1]), K), np.float32)
    for e, c in enumerate(counts):
        A[offs[e]:offs[e] + c] = rng.standard_normal((c, K), dtype=np.float32)
    qA, sA = I.quantize(A)
    qB = np.empty((4, N, K), np.uint8)
    sB = np.empty((4, -(-N // 128), K // 128), np.float32)
    for e in range(4):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    C = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(offs), "f32")
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, offs)
    r = ratio(C.cpu().numpy().astype(np.float64), Cr, mass, "f32")
    print(f"  grouped: max err/bound = {r:.3g}", flush=True)
    worst = max(worst, r)
    return 0 if worst <= 1.0 else 1


if __name__ == "__main__":
    sys.exit(main())
