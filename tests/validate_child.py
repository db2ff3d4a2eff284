"""Child process of tests/test_gpu_overrides.py (not collected by pytest).

Runs with DG_VALIDATE=1, which the library reads once per process: grouped
calls then copy group_offsets to the host and reject offsets that break the
layout rules before launching anything.  Valid offsets must still give
results inside the parity bound; every invalid set must raise.  Exit status
0 when all of that holds."""
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


def main():
    assert os.environ.get("DG_VALIDATE") == "1"
    rng = np.random.default_rng(7)
    G, N, K, M_total = 3, 256, 256, 384
    A = rng.standard_normal((M_total, K), dtype=np.float32)
    qB = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, N // 128, K // 128), np.float32)
    for e in range(G):
        qB[e], sB[e] = I.quantize(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    qA, sA = I.quantize(A)                       # 128 x 128 A scales
    qA1, sA1 = I.quantize(A, rows=1)             # one A scale per row
    ok = True

    good = np.array([0, 128, 128, 384], np.int32)
    C = dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(good), "f32")
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA, sA, qB, sB, good)
    r = float((np.abs(C.cpu().numpy() - Cr) / oracle.tolerance(Cr, mass, "f32")).max())
    print(f"  padded, valid offsets: max err/bound = {r:.3g}", flush=True)
    ok &= r <= 1.0

    packed = np.array([0, 5, 5, 384], np.int32)
    C = dg.grouped_gemm_fp8_segments(t(qA1), t(sA1), t(qB), t(sB), t(packed), "f32")
    torch.cuda.synchronize()
    Cr, mass = oracle.grouped_gemm(qA1, sA1, qB, sB, packed, sa_rows=1)
    r = float((np.abs(C.cpu().numpy() - Cr) / oracle.tolerance(Cr, mass, "f32")).max())
    print(f"  packed, valid offsets: max err/bound = {r:.3g}", flush=True)
    ok &= r <= 1.0

    bad_padded = {"not a multiple of 128": [0, 100, 256, 384], "decreasing": [0, 256, 128, 384],
                  "first not 0": [128, 128, 256, 384], "last not M_total": [0, 128, 256, 256]}
    for why, offs in bad_padded.items():
        try:
            dg.grouped_gemm_fp8(t(qA), t(sA), t(qB), t(sB), t(np.array(offs, np.int32)), "f32")
            print(f"  padded, {why}: accepted (wrong)", flush=True)
            ok = False
        except dg.DGError as exc:
            print(f"  padded, {why}: rejected ({exc})", flush=True)
            ok &= exc.status == dg.DG_ERR_INVALID_ARG
    bad_packed = {"decreasing": [0, 9, 5, 384], "last past M_total": [0, 5, 9, 400]}
    for why, offs in bad_packed.items():
        try:
            dg.grouped_gemm_fp8_segments(t(qA1), t(sA1), t(qB), t(sB), t(np.array(offs, np.int32)), "f32")
            print(f"  packed, {why}: accepted (wrong)", flush=True)
            ok = False
        except dg.DGError as exc:
            print(f"  packed, {why}: rejected ({exc})", flush=True)
            ok &= exc.status == dg.DG_ERR_INVALID_ARG
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
