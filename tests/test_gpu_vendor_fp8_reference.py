"""The numerics behind the choice of the FP16 matrix cores, measured against
the vendor's FP8 GEMM.  torch._scaled_mm (hipBLASLt, E4M3 operands, unit
per-tensor scales, FP32 out) accumulates on gfx950's FP8 matrix cores; with
unit scales it computes exactly the product that the oracle defines for unit
block scales, so its error against the oracle is the FP8 accumulation's own.
The test logs the vendor's max err/bound beside this library's and asserts
only this library's result (the vendor's figure documents the design, it is
not a requirement).  Needs a GPU; skipped when torch has no FP8 GEMM."""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_block_amd import dg

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def ratio(C, Cr, mass):
    Cg = C.float().cpu().numpy().astype(np.float64)
    return float((np.abs(Cg - Cr) / oracle.tolerance(Cr, mass, "f32")).max())


@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (64, 144, 128), (1024, 1024, 1024)])
def test_fp8_matrix_core_accumulation_vs_this_library(M, N, K):
    if not hasattr(torch, "_scaled_mm"):
        pytest.skip("torch has no FP8 GEMM")
    rng = np.random.default_rng(M + K)
    A = torch.from_numpy(rng.standard_normal((M, K), dtype=np.float32)).to(torch.float8_e4m3fn)
    B = torch.from_numpy(rng.standard_normal((N, K), dtype=np.float32)).to(torch.float8_e4m3fn)
    qa, qb = A.view(torch.uint8).numpy(), B.view(torch.uint8).numpy()
    sA = np.ones((-(-M // 128), K // 128), np.float32)
    sB = np.ones((-(-N // 128), K // 128), np.float32)
    one = torch.ones((), device=DEV)
    try:
        Cv = torch._scaled_mm(A.to(DEV), B.to(DEV).t(), scale_a=one, scale_b=one, out_dtype=torch.float32)
    except RuntimeError as e:      # pragma: no cover - depends on the torch build
        pytest.skip(f"torch._scaled_mm unavailable here: {e}")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    Cd = dg.gemm_fp8_blockscaled(t(qa), t(sA), t(qb), t(sB), "f32")
    torch.cuda.synchronize()
    Cr, mass = oracle.gemm_blockscaled(qa, sA, qb, sB)
    rv, rd = ratio(Cv, Cr, mass), ratio(Cd, Cr, mass)
    print(f"  {M}x{N}x{K} FP32 out: vendor FP8 GEMM max err/bound = {rv:.3g}, this library = {rd:.3g}",
          file=sys.stderr, flush=True)
    assert rd <= 1.0
