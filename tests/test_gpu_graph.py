"""The library under HIP graph capture: a chain of dependent calls
(quantise -> GEMM -> quantise -> GEMM -> quantise -> grouped GEMM) captured
once and replayed several times must reproduce the eager chain bit for bit.
Intermediate buffers are poisoned with NaN / 0xFF between replays, so a call
that started before the one producing its input would be caught.  Needs a
GPU."""
import sys

import numpy as np
import pytest
import torch

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


def test_dependent_chain_replays_match_eager():
    log("graph chain: quantise -> gemm -> quantise -> gemm -> quantise -> segments")
    rng = np.random.default_rng(12)
    M, D = 1024, 2048
    x = torch.from_numpy(rng.standard_normal((M, D)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    w = []
    for _ in range(2):
        q, s = I.quantize((rng.standard_normal((D, D)) * 0.03).astype(np.float32))
        w.append((torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV)))
    G = 8
    counts = rng.multinomial(M, np.full(G, 1.0 / G))
    counts[3] += counts[5]
    counts[5] = 0                                 # an empty expert
    offs_np = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    qe, se = I.quantize((rng.standard_normal((G * D, D)) * 0.03).astype(np.float32))
    qe, se = qe.reshape(G, D, D), se.reshape(G, D // 128, D // 128)
    qe, se, offs = torch.from_numpy(qe).to(DEV), torch.from_numpy(se).to(DEV), torch.from_numpy(offs_np).to(DEV)

    Q = [torch.empty((M, D), dtype=torch.uint8, device=DEV) for _ in range(3)]
    S = [torch.empty((M, D // 128), dtype=torch.float32, device=DEV),
         torch.empty((M // 128, D // 128), dtype=torch.float32, device=DEV),
         torch.empty((M, D // 128), dtype=torch.float32, device=DEV)]
    C = [torch.empty((M, D), dtype=torch.bfloat16, device=DEV) for _ in range(3)]

    def chain():
        dg.quantize_fp8_blockscaled(x, 1, Q=Q[0], S=S[0])
        dg.gemm_fp8_blockscaled(Q[0], S[0], w[0][0], w[0][1], "bf16", C=C[0])
        dg.quantize_fp8_blockscaled(C[0], 128, Q=Q[1], S=S[1])
        dg.gemm_fp8_blockscaled(Q[1], S[1], w[1][0], w[1][1], "bf16", C=C[1])
        dg.quantize_fp8_blockscaled(C[1], 1, Q=Q[2], S=S[2])
        dg.grouped_gemm_fp8_segments(Q[2], S[2], qe, se, offs, "bf16", C=C[2])

    def poison():
        for t in Q:
            t.fill_(0xFF)                        # E4M3 NaN codes
        for t in S + C:
            t.fill_(float("nan"))

    poison()
    chain()
    torch.cuda.synchronize()
    want = [t.clone() for t in Q + S + C]
    assert all(bool(torch.isfinite(t.float()).all()) for t in S + C)

    g = torch.cuda.CUDAGraph()
    poison()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=torch.cuda.Stream()):
        chain()
    torch.cuda.synchronize()
    for rep in range(4):
        poison()                                 # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = Q + S + C
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: buffer {i} differs from the eager chain"
        log(f"  replay {rep}: all {len(got)} buffers match the eager chain")


def test_noalloc_call_captured_in_a_graph():
    """dg_gemm_fp8_ex_noalloc captured on a stream that has never run a
    library call (so no workspace exists for it): the split of K uses the
    static scratch, and four replays, with eager work in between, equal the
    eager dg_gemm_fp8_ex result bit for bit."""
    M, N, K = 256, 4096, 4096                     # K split 4 ways
    p = I.dense_problem(M, N, K, seed=21, out_dtype="bf16", block_log2_range=3.0)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    A, sA, B, sB = t(p.A), t(p.sA), t(p.B), t(p.sB)
    want = dg.gemm_fp8_blockscaled(A, sA, B, sB, "bf16")
    torch.cuda.synchronize()
    C = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    args = (A.data_ptr(), 0, sA.data_ptr(), 128, B.data_ptr(), 0, sB.data_ptr(), C.data_ptr(), M, N, K,
            dg.DG_OUT_BF16)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=s):
        st = dg.dg_gemm_fp8_ex_noalloc(*args, torch.cuda.current_stream().cuda_stream)
    assert st == dg.DG_OK, dg.dg_status_string(st)
    for rep in range(4):
        C.fill_(float("nan"))
        dg.gemm_fp8_blockscaled(A, sA, B, sB, "bf16")   # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(C, want), f"replay {rep} differs from the eager result"
    log("  noalloc call captured in a graph: 4 replays equal the eager result")

