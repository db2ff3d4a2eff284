"""dg_gemm_fp8_ex_noalloc: the allocation-free variant of dg_gemm_fp8_ex whose
split-K partials go to the library's static device scratch instead of a
per-stream workspace.

GPU: two calls in a row through the C-ABI, the second with a smaller input,
each compared with dg_gemm_fp8_ex on the same operands (the same kernels and
the same split of K: bit-identical) and with the CPU oracle at the parity
bound.  Both shapes are split (on the MI355X's 256 CUs: 4 and 2 ways), so the
scratch is written and read by both calls, the second over what the first
left there.
CPU: host-side argument errors match dg_gemm_fp8_ex's, and a split that the
DG_SPLITK override makes larger than the scratch is rejected before any HIP
call (child process: the override is read once per process)."""
import ctypes
import os
import subprocess
import sys

import numpy as np
import pytest

import parity_log

import oracle
from moe_grouped_gemm_block_amd import dg
from moe_grouped_gemm_block_amd import inputs as I

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
P = 1 << 20                                   # a 16-byte aligned fake address (never dereferenced)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def raw(fn, A, sA, B, sB, C, M, N, K, out=1, fa=0, fb=0, rows=128, stream=None):
    return fn(A, fa, sA, rows, B, fb, sB, C, M, N, K, out, stream)


@pytest.mark.parametrize("kw,want", [
    (dict(A=None), dg.DG_ERR_INVALID_ARG), (dict(K=200), dg.DG_ERR_UNSUPPORTED),
    (dict(out=3), dg.DG_ERR_INVALID_ARG), (dict(M=0), dg.DG_OK), (dict(sA=P + 2), dg.DG_ERR_INVALID_ARG),
    (dict(rows=64), dg.DG_ERR_INVALID_ARG), (dict(fa=2), dg.DG_ERR_INVALID_ARG),
])
def test_noalloc_host_errors_match_ex(kw, want):
    d = dict(A=P, sA=P, B=P, sB=P, C=P, M=256, N=256, K=256, out=1, fa=0, fb=0, rows=128)
    d.update(kw)
    assert raw(dg.dg_gemm_fp8_ex_noalloc, **d) == want
    assert raw(dg.dg_gemm_fp8_ex, **d) == want


def test_noalloc_rejects_a_split_larger_than_the_scratch():
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from moe_grouped_gemm_block_amd import dg\n"
            "P = 1 << 20\n"
            # 8 splits of 4096 x 4096 FP32 partials = 512 MB > 32 MB
            "st = dg.dg_gemm_fp8_ex_noalloc(P, 0, P, 128, P, 0, P, P, 4096, 4096, 4096, 1, None)\n"
            "print(st, dg.dg_status_string(st))\n"
            "sys.exit(0 if st == dg.DG_ERR_UNSUPPORTED else 1)\n") % ROOT
    env = dict(os.environ, DG_SPLITK="8")
    env.pop("DG_FORCE_TILE", None)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    log(r.stdout.strip())
    assert r.returncode == 0, r.stdout + r.stderr[-2000:]
    assert "32 MB static scratch" in r.stdout


@pytest.mark.gpu
def test_noalloc_matches_ex_two_calls():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dev = "cuda:0"
    stream = torch.cuda.current_stream().cuda_stream
    # second call smaller than the first; both split K (4 and 2 ways)
    for (M, N, K, out) in [(256, 4096, 4096, "bf16"), (136, 1000, 2048, "f32")]:
        log(f"noalloc {M}x{N}x{K} {out}")
        p = I.dense_problem(M, N, K, seed=M + N + K, out_dtype=out, block_log2_range=3.0)
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
        A, sA, B, sB = t(p.A), t(p.sA), t(p.B), t(p.sB)
        cdt = torch.bfloat16 if out == "bf16" else torch.float32
        C_ex = torch.full((M, N), float("nan"), dtype=cdt, device=dev)
        C_na = torch.full((M, N), float("nan"), dtype=cdt, device=dev)
        code = dg.out_code(out)
        args = (A.data_ptr(), 0, sA.data_ptr(), 128, B.data_ptr(), 0, sB.data_ptr())
        st = dg.dg_gemm_fp8_ex_noalloc(*args, C_na.data_ptr(), M, N, K, code, stream)
        assert st == dg.DG_OK, dg.dg_status_string(st)
        st = dg.dg_gemm_fp8_ex(*args, C_ex.data_ptr(), M, N, K, code, stream)
        assert st == dg.DG_OK, dg.dg_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(C_na, C_ex), "noalloc result differs from dg_gemm_fp8_ex"
        Cg = C_na.float().cpu().numpy().astype(np.float64)
        Cr, mass = oracle.gemm_blockscaled(p.A, p.sA, p.B, p.sB)
        bound = oracle.tolerance(Cr, mass, out)
        ratio = float((np.abs(Cg - Cr) / bound).max())
        log(f"  noalloc {M}x{N}x{K} {out}: max err/bound = {ratio:.3g}")
        parity_log.record(f"noalloc {M}x{N}x{K} {out}", ratio)
        assert ratio <= 1.0
