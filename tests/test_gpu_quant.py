"""Parity of the HIP activation quantisation (through the C-ABI) with the CPU
oracle.  Needs a GPU.  Codes and scales are integer / byte results of a
float decision taken in the same precision on both sides (double quotient),
so the bar is bit-exact equality."""
import sys

import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_block_amd import dg

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    dg.lib()


def run(x32: np.ndarray, dtype: str, R: int):
    """Quantise on the GPU; returns (codes, scales, the float32 values the GPU saw)."""
    t = torch.from_numpy(np.ascontiguousarray(x32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    seen = t.float().numpy()
    Q, S = dg.quantize_fp8_blockscaled(t.to(DEV), block_rows=R)
    torch.cuda.synchronize()
    return Q.cpu().numpy(), S.cpu().numpy(), seen


def check(x32, dtype, R, rows=None, what=""):
    q, s, seen = run(x32, dtype, R)
    if rows is not None:                      # R = 1: rows are independent
        assert R == 1
        seen, q, s = seen[rows], q[rows], s[rows]
    qo, so = oracle.quantize_blockscaled(seen, R)
    bad_s = np.argwhere(s.view(np.uint32) != so.view(np.uint32))
    bad_q = np.argwhere(q != qo)
    log(f"  {what}: {bad_q.shape[0]} code and {bad_s.shape[0]} scale mismatches")
    assert bad_s.shape[0] == 0, (bad_s[:5].tolist(), s.flat[:3], so.flat[:3])
    assert bad_q.shape[0] == 0, [(tuple(i), int(q[tuple(i)]), int(qo[tuple(i)])) for i in bad_q[:5]]


SHAPES = [(1, 128), (5, 256), (127, 256), (128, 128), (129, 384), (300, 1024)]


@pytest.mark.parametrize("R", [128, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K", SHAPES)
def test_quantize_random(M, K, dtype, R):
    rng = np.random.default_rng(M * 31 + K + R)
    x = (rng.standard_normal((M, K)) * np.exp2(rng.uniform(-6, 6, (M, 1)))).astype(np.float32)
    x[rng.random((M, K)) < 0.01] *= 50.0       # outliers
    log(f"quantize M={M} K={K} {dtype} R={R}")
    check(x, dtype, R, what=f"{M}x{K} {dtype} R={R}")


@pytest.mark.parametrize("R", [128, 1])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_special_values(dtype, R):
    """Exact ties (block amax 448 gives s = 1, so x / s is every E4M3 midpoint
    exactly), -0, zeros, an all-zero block, tiny and huge magnitudes."""
    vals = oracle.decode_table()[:0x7F]
    mids = (vals[1:] + vals[:-1]) / 2                       # 126 midpoints, exact in bf16
    M, K = 130, 384
    x = np.zeros((M, K), np.float32)
    for r in range(M):
        row = np.concatenate([mids, -mids, [448.0, -0.0]]).astype(np.float32)
        x[r, :128] = np.roll(row[:128], r)
        x[r, 127] = 448.0                                   # every 1 x 128 block: amax 448
    x[:, 128:256] = 0.0                                      # all-zero blocks
    x[:, 128 + 5] = -0.0
    tiny = np.float32(2.0 ** -120)
    x[:, 256:384] = np.float32(3e30)
    x[::3, 256:384] = tiny
    x[1, 300] = -1e-38                                       # subnormal input
    log(f"quantize special values {dtype} R={R}")
    check(x, dtype, R, what=f"special {dtype} R={R}")


@pytest.mark.parametrize("R", [128, 1])
def test_quantize_full_size_bf16(R):
    """The 4096 x 4096 activation of the dense workload, BF16 in."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4096, 4096)).astype(np.float32)
    mult = np.exp2(rng.uniform(-4, 4, (32, 32))).astype(np.float32)   # per-block magnitudes
    x *= np.repeat(np.repeat(mult, 128, axis=0), 128, axis=1)
    log(f"quantize 4096x4096 bf16 R={R}")
    if R == 128:
        check(x, "bf16", R, what="4096^2 R=128")
    else:
        rows = np.unique(np.concatenate([np.arange(64), rng.integers(0, 4096, 64), [4095]]))
        check(x, "bf16", R, rows=rows, what="4096^2 R=1 sampled rows")


def test_quantize_repeatable():
    rng = np.random.default_rng(4)
    x = torch.from_numpy(rng.standard_normal((512, 1024)).astype(np.float32)).to(DEV)
    q1, s1 = dg.quantize_fp8_blockscaled(x, 128)
    q2, s2 = dg.quantize_fp8_blockscaled(x, 128)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


def test_quantized_operand_feeds_the_gemm():
    """GPU-quantised A and B go straight into the GEMM; the result matches the
    oracle GEMM on the oracle's own codes and scales of the same inputs."""
    rng = np.random.default_rng(8)
    M, N, K = 200, 264, 512
    a = rng.standard_normal((M, K)).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, sa = dg.quantize_fp8_blockscaled(torch.from_numpy(a).to(DEV), 128)
    qb, sb = dg.quantize_fp8_blockscaled(torch.from_numpy(b).to(DEV), 128)
    C = dg.gemm_fp8_blockscaled(qa, sa, qb, sb, "f32")
    torch.cuda.synchronize()
    qao, sao = oracle.quantize_blockscaled(a, 128)
    qbo, sbo = oracle.quantize_blockscaled(b, 128)
    Cr, mass = oracle.gemm_blockscaled(qao, sao, qbo, sbo)
    err = np.abs(C.cpu().numpy().astype(np.float64) - Cr)
    assert np.all(err <= oracle.tolerance(Cr, mass, "f32"))


@pytest.mark.parametrize("R", [128, 1])
def test_quantize_writes_nothing_outside_q_and_s(R):
    """Q and S are views into larger buffers filled with a marker: the bytes
    before and after them are untouched (ragged M, several K-blocks)."""
    log(f"quantize guard bands R={R}")
    rng = np.random.default_rng(9)
    M, K = 131, 384
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    G = 256
    qbuf = torch.full((M * K + 2 * G,), 0x5A, dtype=torch.uint8, device=DEV)
    ns = -(-M // R) * (K // 128)
    sbuf = torch.full((ns + 2 * 64,), 7.0, dtype=torch.float32, device=DEV)
    Q = qbuf[G:G + M * K].view(M, K)
    S = sbuf[64:64 + ns].view(-(-M // R), K // 128)
    dg.quantize_fp8_blockscaled(x, R, Q=Q, S=S)
    torch.cuda.synchronize()
    qb, sb = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.all(qb[:G] == 0x5A) and np.all(qb[G + M * K:] == 0x5A)
    assert np.all(sb[:64] == 7.0) and np.all(sb[64 + ns:] == 7.0)
    qo, so = oracle.quantize_blockscaled(x.float().cpu().numpy(), R)
    assert np.array_equal(Q.cpu().numpy(), qo) and np.array_equal(S.cpu().numpy(), so)
