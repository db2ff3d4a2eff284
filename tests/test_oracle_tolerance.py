"""Pins of the oracle's pass test, oracle.tolerance() (CPU only).

Every GPU parity test and the smoke check decide pass / fail with
oracle.tolerance(C_ref, mass, out_dtype).  The bound is the one the task
states for an FP32-accumulating device (block partials accumulated in FP32,
FP8-for-MoE page 2kiu.com/news/5461879, section 3.3):

    FP32 output:  |C_gpu - C_ref| <= 1e-5 * mass + 1e-6
    BF16 output:  the same plus 2^-8 * |C_ref| (the final rounding to BF16)

with mass = sum |a b sA sB|.  A loosened bound would let real accumulation
bugs pass everywhere, a tightened one would reject correct FP32 arithmetic.
The checks below fix it from outside the function:

* hand-computed values of the formula;
* it admits what a correct device does: a float32 emulation of the
  block-scaled product (exact block partials or sequential FP32 sums, FP32
  rescale-FMA per K-block), and the round-to-nearest-even conversion to BF16
  done by a library cast;
* it rejects emulated devices with the accumulation bugs this path could
  plausibly have: BF16-precision accumulation, FP8-matrix-core-style
  truncation of small products inside groups of 8, a dropped last K-element,
  BF16 rounding on an FP32 output, and a uniform error of 2e-5 * mass;
* loosened and tightened variants of the function, put in its place, fail
  at least one of these checks.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import blockscaled as OB

KB = 128


# --------------------------------------------------------------------------- emulated devices
# Independent of the oracle's arithmetic: operands decoded by torch's
# float8_e4m3fn cast, arithmetic in numpy float32 (products of two E4M3
# values have at most 8 significant bits, so they are exact in float32).

def lib_decode(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def device(A, sA, B, sB, partial="exact", acc_round=None, drop_last_k=False, trunc8=False):
    """C[M][N] of an emulated device, float64 array of float32 values.

    partial: "exact" (block partial summed exactly, then rounded once to
    float32, as a wide-window matrix core does) or "seq" (sequential float32
    sum over the block).  acc_round: None or "bf16" (accumulator rounded to
    BF16 after every K-block).  drop_last_k: the last K element is never
    added.  trunc8: inside each group of 8 consecutive K elements, products
    below 2^(e_max - 13) of the group's largest product are dropped (the
    behaviour measured on gfx950's FP8 matrix-core instruction).
    """
    a = lib_decode(A).astype(np.float64)
    b = lib_decode(B).astype(np.float64)
    M, K = a.shape
    N = b.shape[0]
    Kb = -(-K // KB)
    acc = np.zeros((M, N), np.float32)
    for kb in range(Kb):
        lo, hi = kb * KB, min(K, (kb + 1) * KB)
        if drop_last_k and hi == K:
            hi -= 1
        prods = a[:, None, lo:hi] * b[None, :, lo:hi]            # exact, [M][N][k]
        if trunc8:
            for g in range(0, hi - lo, 8):
                grp = prods[:, :, g:g + 8]
                mx = np.abs(grp).max(axis=2, keepdims=True)
                with np.errstate(divide="ignore"):
                    floor = np.where(mx > 0, np.exp2(np.floor(np.log2(np.where(mx > 0, mx, 1))) - 13), 0)
                grp[np.abs(grp) < floor] = 0.0
        if partial == "exact":
            P = prods.sum(axis=2).astype(np.float32)
        else:
            P = np.zeros((M, N), np.float32)
            for k in range(prods.shape[2]):
                P = (P + prods[:, :, k].astype(np.float32)).astype(np.float32)
        s = (sA[np.arange(M) // KB, kb][:, None].astype(np.float32)
             * sB[np.arange(N) // KB, kb][None, :].astype(np.float32)).astype(np.float32)
        acc = (s.astype(np.float64) * P + acc).astype(np.float32)      # one rounding, like an FMA
        if acc_round == "bf16":
            acc = torch.from_numpy(acc).to(torch.bfloat16).float().numpy()
    return acc.astype(np.float64)


def to_bf16(C):
    return torch.from_numpy(C.astype(np.float32)).to(torch.bfloat16).double().numpy()


def problem(seed, M=32, N=48, K=512, spread=4.0):
    """Gaussian data with a per-128x128-block magnitude 2^U(-spread, spread),
    quantised by the shared generator (amax/448 scales, RNE to E4M3)."""
    from moe_grouped_gemm_block_amd import inputs as I
    p = I.dense_problem(M, N, K, seed=seed, out_dtype="f32", block_log2_range=spread)
    return p.A, p.sA, p.B, p.sB


def positive_problem(M=8, N=8, K=2048, seed=11):
    """Positive Gaussian magnitudes (no cancellation anywhere), quantised by
    the shared generator."""
    from moe_grouped_gemm_block_amd import inputs as I
    rng = np.random.default_rng(seed)
    qa, sa = I.quantize(np.abs(rng.standard_normal((M, K), dtype=np.float32)))
    qb, sb = I.quantize(np.abs(rng.standard_normal((N, K), dtype=np.float32)))
    return qa, sa, qb, sb


def crafted_window_case():
    """One output whose only K-group holds a product of 2^16 and seven of 2^2:
    a device that truncates below 2^(16-13) loses 28 of a mass of 65564."""
    def code(v):
        return torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    K = KB
    A = np.zeros((1, K), np.uint8)
    B = np.zeros((1, K), np.uint8)
    A[0, 0], B[0, 0] = code(256.0), code(256.0)
    A[0, 1:8], B[0, 1:8] = code(2.0), code(2.0)
    one = np.ones((1, 1), np.float32)
    return A, one, B, one


# --------------------------------------------------------------------------- the checks

def pin_failures(tol):
    """Run every pin against the tolerance function `tol`; return the names
    of the pins it fails."""
    bad = []

    # 1. hand-computed values
    C = np.array([1.0, -256.0, 0.0, 3.0e4])
    mass = np.array([0.0, 1.0e5, 3.0, 3.0e4])
    want_f32 = np.array([1e-6, 1.0 + 1e-6, 3e-5 + 1e-6, 0.3 + 1e-6])
    want_bf16 = want_f32 + np.array([2.0 ** -8, 1.0, 0.0, 3.0e4 / 256])
    if not np.allclose(tol(C, mass, "f32"), want_f32, rtol=1e-12, atol=0):
        bad.append("hand values f32")
    if not np.allclose(tol(C, mass, "bf16"), want_bf16, rtol=1e-12, atol=0):
        bad.append("hand values bf16")

    # 2. the FP32 bound does not depend on C (the 2^-8 term is for BF16 only)
    m = np.full(5, 10.0)
    if not np.array_equal(tol(np.zeros(5), m, "f32"), tol(np.full(5, 1e6), m, "f32")):
        bad.append("f32 bound depends on C")

    # 3. a uniform error of 2e-5 * mass on FP32 output is out of bound
    mass = np.array([1.0, 10.0, 1e3, 1e6])
    if np.any(tol(np.zeros(4), mass, "f32") >= 2e-5 * mass):
        bad.append("2e-5*mass accepted on f32")

    # 4. correct FP32 devices pass, on three seeds with block magnitudes
    for seed in (1, 2, 3):
        A, sA, B, sB = problem(seed)
        Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB)
        for partial in ("exact", "seq"):
            Cg = device(A, sA, B, sB, partial=partial)
            if np.any(np.abs(Cg - Cr) > tol(Cr, mass, "f32")):
                bad.append(f"correct fp32 device ({partial}) rejected, seed {seed}")
            # BF16 output by a library cast (round to nearest even)
            if np.any(np.abs(to_bf16(Cg) - Cr) > tol(Cr, mass, "bf16")):
                bad.append(f"correct bf16 output rejected, seed {seed}")

    # 4b. no cancellation: positive operands, sequential FP32 block sums over
    #     K = 2048 (errors of a few 1e-6 * mass, which the bound must admit;
    #     a bound a hundred times tighter would reject this correct device)
    A, sA, B, sB = positive_problem()
    Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    Cg = device(A, sA, B, sB, partial="seq")
    err = np.abs(Cg - Cr)
    if np.any(err > tol(Cr, mass, "f32")):
        bad.append("correct fp32 device (seq, positive data) rejected")
    if not np.any(err > 1e-7 * mass + 1e-6):
        bad.append("positive-data case not sharp")

    # 5. the BF16 term covers the worst round-to-nearest case: values just
    #    above a power of two, whose rounding error is half an ulp, almost
    #    2^-8 of the value (mass 0: nothing else to absorb it)
    x = np.ldexp(1.0 + 2.0 ** -8 - 2.0 ** -23, np.arange(-20, 20)).astype(np.float32).astype(np.float64)
    x = np.concatenate([x, -x])
    r = to_bf16(x)
    if np.any(np.abs(r - x) > tol(x, np.zeros_like(x), "bf16")):
        bad.append("bf16 rounding of near-ties rejected")
    if not np.all(np.abs(r - x) > 0.99 * 2.0 ** -8 * np.abs(x)):   # the cases are as bad as claimed
        bad.append("near-tie cases not sharp")

    # 5b. a conversion to BF16 that truncates instead of rounding is out of
    #     bound just above a power of two (its error there is almost 2^-7)
    x = np.ldexp(1.0 + 2.0 ** -7 - 2.0 ** -23, np.arange(-20, 20)).astype(np.float32)
    t = (x.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    x = x.astype(np.float64)
    if np.all(np.abs(t - x) <= tol(x, np.zeros_like(x), "bf16")):
        bad.append("truncating bf16 conversion accepted")

    # 6. buggy devices are rejected
    A, sA, B, sB = problem(7, M=32, N=48, K=1024)
    Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    Cg = device(A, sA, B, sB, acc_round="bf16")
    if np.all(np.abs(Cg - Cr) <= tol(Cr, mass, "f32")):
        bad.append("bf16-accumulating device accepted (f32 out)")
    if np.all(np.abs(to_bf16(Cg) - Cr) <= tol(Cr, mass, "bf16")):
        bad.append("bf16-accumulating device accepted (bf16 out)")
    Cg = device(A, sA, B, sB, drop_last_k=True)
    if np.all(np.abs(Cg - Cr) <= tol(Cr, mass, "f32")):
        bad.append("device dropping the last K element accepted")
    Cg = to_bf16(device(A, sA, B, sB))                               # BF16 result handed out as FP32
    if np.all(np.abs(Cg - Cr) <= tol(Cr, mass, "f32")):
        bad.append("bf16-rounded result accepted as f32")
    A, sA, B, sB = crafted_window_case()
    Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    Cg = device(A, sA, B, sB, trunc8=True)
    if np.all(np.abs(Cg - Cr) <= tol(Cr, mass, "f32")):
        bad.append("FP8-window truncating device accepted")
    return bad


# --------------------------------------------------------------------------- tests

def test_emulated_devices_do_what_they_claim():
    """The emulations themselves: the correct device is exact on the crafted
    window case, the truncating one loses exactly the seven products of 4."""
    A, sA, B, sB = crafted_window_case()
    assert device(A, sA, B, sB)[0, 0] == 65536 + 28
    assert device(A, sA, B, sB, trunc8=True)[0, 0] == 65536
    Cr, mass = oracle.gemm_blockscaled(A, sA, B, sB)
    assert Cr[0, 0] == 65564 and mass[0, 0] == 65564


def test_tolerance_meets_every_pin():
    assert pin_failures(oracle.tolerance) == []


def _loose_mass(C, mass, out):                     # 1e-4 instead of 1e-5
    b = 1e-4 * mass + 1e-6
    return b + 2.0 ** -8 * np.abs(C) if out == "bf16" else b


def _bf16_term_always(C, mass, out):               # 2^-8 |C| applied to FP32 too
    return 1e-5 * mass + 1e-6 + 2.0 ** -8 * np.abs(C)


def _loose_rel(C, mass, out):                      # 2^-7 for the BF16 term
    b = 1e-5 * mass + 1e-6
    return b + 2.0 ** -7 * np.abs(C) if out == "bf16" else b


def _no_abs_term(C, mass, out):                    # the 1e-6 floor dropped
    b = 1e-5 * mass
    return b + 2.0 ** -8 * np.abs(C) if out == "bf16" else b


def _no_bf16_term(C, mass, out):                   # BF16 output held to the FP32 bound
    return 1e-5 * mass + 1e-6


def _tight_mass(C, mass, out):                     # 1e-7: rejects correct FP32 arithmetic
    b = 1e-7 * mass + 1e-6
    return b + 2.0 ** -8 * np.abs(C) if out == "bf16" else b


@pytest.mark.parametrize("variant", [_loose_mass, _bf16_term_always, _loose_rel, _no_abs_term,
                                     _no_bf16_term, _tight_mass])
def test_wrong_tolerances_fail_a_pin(variant, monkeypatch):
    """Planted slips: each variant, put in place of oracle.tolerance, fails
    at least one pin."""
    monkeypatch.setattr(OB, "tolerance", variant)
    monkeypatch.setattr(oracle, "tolerance", variant)
    assert pin_failures(oracle.tolerance) != []
