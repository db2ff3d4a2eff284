"""CPU oracle for FP8 (E4M3) GEMM with 128x128 block scales -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  The product path (the HIP library and its Python binding) never
imports it, and it imports nothing from the product path.

What it computes (plain definition, float64, no blocking or fusion beyond the
definition itself):

    C[i, j] = sum over K-blocks kb of
              sA[i // 128, kb] * sB[j // 128, kb]
              * sum_{k in block kb} dec(A[i, k]) * dec(B[j, k])

Sources:
  * Block-wise scaling: A (M x K) and B (K x N) are cut into blocks, e.g.
    128 x 128, each with one factor, and each output block is multiplied by
    the matching A-block and B-block factors -- DeepGEMM FP8-for-MoE page
    (2kiu.com/news/5461879), section 2.1.  Because the factors vary along K,
    the only reading that is exact is to apply sA*sB to each K-block's
    partial sum before adding it into the FP32 (here: float64) accumulator;
    that page's section 3.3 speaks of FP32 accumulation and segmented
    accumulation.
  * E4M3 layout (1 sign, 4 exponent, 3 mantissa bits, max 448): DeepGEMM FP8
    kernel write-up (demingchina.com/news/60142), section 3.1 table.  The OCP
    E4M3FN variant (exponent bias 7, no infinities, S.1111.111 = NaN) is the
    one whose largest finite value is 448.
  * Layout: A row-major, B column-major (stored N x K, K contiguous), the
    caller supplies both scale sets -- FP8-for-MoE page, section 4.3.
  * MoE grouped variant: every expert's rows sit in one contiguous matrix,
    one segment per expert -- nxmr.cn/news/132300, section 2.2.
  * Per-row A scales (sa_rows = 1): the granularity table of the FP8 kernel
    write-up (demingchina.com/news/60142, section 5.2) lists groups of 128
    elements; for A that is one factor per row and 128-wide K-block, and the
    definition above then reads sA[i, kb] in place of sA[i // 128, kb].

Exactness: every E4M3 value is an integer multiple of 2^-9 below 2^9, so a
product is a multiple of 2^-18 below 2^18 and a sum of up to 2^12 products
needs at most 48 significant bits: each K-block partial is exact in float64
whatever the summation order (BLAS included).  fp32 * fp32 scale products are
exact in float64 too.  The only roundings are one per K-block (the scaled
partial) plus one per addition, so |C_oracle - C_exact| <= (Kb + 1) * 2^-53 * mass.

Parity pins: see tests/test_oracle_pins.py (exhaustive decode against the
format's bit definition and a library cast, exact rational brute force,
integer closed forms, identity / permutation, K-block reordering, scale
homogeneity, transposition symmetry, grouped == per-expert dense).
"""
from __future__ import annotations

import numpy as np

BLOCK = 128


def e4m3_value(code: int) -> float:
    """Value of one OCP E4M3FN byte, from its bit fields.

    sign = bit 7, exponent field e = bits 6..3 (bias 7), mantissa m = bits 2..0.
    e == 0: subnormal, m * 2^-9 (= m/8 * 2^-6).  e == 15 and m == 7: NaN.
    Otherwise (1 + m/8) * 2^(e - 7).
    """
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e5m2_value(code: int) -> float:
    """Value of one E5M2 byte, from its bit fields (the FP8 kernel write-up's
    section 3.1 table: 1 sign, 5 exponent, 2 mantissa bits).

    sign = bit 7, exponent field e = bits 6..2 (bias 15), mantissa m = bits 1..0.
    e == 0: subnormal, m * 2^-16 (= m/4 * 2^-14).  e == 31: infinity (m == 0)
    or NaN.  Otherwise (1 + m/4) * 2^(e - 15); the largest finite value is
    1.75 * 2^15 = 57344.
    """
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 2) & 0x1F
    m = code & 0x3
    if e == 0x1F:
        return sign * float("inf") if m == 0 else float("nan")
    if e == 0:
        return sign * m * 2.0 ** -16
    return sign * (1.0 + m / 4.0) * 2.0 ** (e - 15)


FORMATS = {"e4m3": e4m3_value, "e5m2": e5m2_value}


def decode_table(fmt: str = "e4m3") -> np.ndarray:
    """float64 [256]: value of every code of the format ("e4m3" = OCP E4M3FN,
    "e5m2")."""
    return np.array([FORMATS[fmt](c) for c in range(256)], dtype=np.float64)


_LUTS = {f: decode_table(f) for f in FORMATS}
_LUT = _LUTS["e4m3"]


def decode(codes: np.ndarray, fmt: str = "e4m3") -> np.ndarray:
    """uint8 codes -> float64 values by table lookup."""
    return _LUTS[fmt][np.asarray(codes, dtype=np.uint8)]


def gemm_blockscaled(A: np.ndarray, sA: np.ndarray, B: np.ndarray, sB: np.ndarray,
                     rows: np.ndarray | None = None,
                     cols: np.ndarray | None = None,
                     a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                     sa_rows: int = 128) -> tuple[np.ndarray, np.ndarray]:
    """Dense block-scaled GEMM.

    A: uint8 [M][K] (row-major), sA: fp32 [ceil(M/sa_rows)][ceil(K/128)]
    B: uint8 [N][K] (B column-major), sB: fp32 [ceil(N/128)][ceil(K/128)]
    When K is not a multiple of 128 the last K-block holds the remaining
    K mod 128 columns and has its own scales, like a partial edge block in M
    or N (the FP8 kernel write-up, section 6, on the K tail).
    rows / cols: optional index subsets of the output to evaluate.
    a_fmt / b_fmt: "e4m3" (default) or "e5m2" codes.
    sa_rows: rows of A per scale block: 128 (128 x 128 blocks) or 1 (one
    scale per row and 128 columns, the 1 x 128 granularity of the FP8 kernel
    write-up, demingchina.com/news/60142, section 5.2 table).  Row i of the
    output then takes A scale sA[i // sa_rows, kb] for K-block kb.

    With an E5M2 operand a block partial can need more than 53 bits (E5M2
    values span 2^-16 .. 57344), so it is then exact only up to BLAS's
    summation error, at most 128 * 2^-53 of the block's sum |a b| -- far
    inside the comparison tolerance.

    Returns (C, mass), both float64 [len(rows)][len(cols)], where
    mass[i, j] = sum_k |dec(A[i,k]) * dec(B[j,k])| * sA * sB (the magnitude the
    tolerance is measured against).
    """
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError("A and B must share K")
    if sa_rows not in (1, BLOCK):
        raise ValueError("sa_rows must be 1 or 128")
    Kb = -(-K // BLOCK)                  # the last K-block may be partial (K tail)
    rows = np.arange(M) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    A64 = decode(A[rows], a_fmt)                              # [m][K]
    B64 = decode(B[cols], b_fmt)                              # [n][K]
    C = np.zeros((len(rows), len(cols)), np.float64)
    mass = np.zeros_like(C)
    for kb in range(Kb):
        ks = slice(kb * BLOCK, min(K, (kb + 1) * BLOCK))
        a = A64[:, ks]
        b = B64[:, ks]
        partial = a @ b.T                                      # exact for E4M3 x E4M3
        absum = np.abs(a) @ np.abs(b).T                        # exact
        scale = (sA[rows // sa_rows, kb].astype(np.float64)[:, None]
                 * sB[cols // BLOCK, kb].astype(np.float64)[None, :])
        C += scale * partial
        mass += scale * absum
    return C, mass


def grouped_gemm(A: np.ndarray, sA: np.ndarray, B: np.ndarray, sB: np.ndarray,
                 group_offsets: np.ndarray,
                 rows: np.ndarray | None = None,
                 cols: np.ndarray | None = None,
                 a_fmt: str = "e4m3", b_fmt: str = "e4m3",
                 sa_rows: int = 128) -> tuple[np.ndarray, np.ndarray]:
    """MoE grouped block-scaled GEMM over contiguous expert segments.

    A: uint8 [M_total][K]; sA: fp32 [M_total/sa_rows][K/128] (sa_rows 128 or 1)
    B: uint8 [G][N][K];    sB: fp32 [G][ceil(N/128)][K/128]
    group_offsets: int [G+1], rows [o_e, o_{e+1}) belong to expert e; the o_e
    are multiples of 128 for 128-row A scale blocks and arbitrary for sa_rows = 1
    (packed segments, as in a decode step with few tokens per expert).
    Each expert's rows are a dense product with that expert's B and sB.
    """
    M_total = A.shape[0]
    G = B.shape[0]
    off = np.asarray(group_offsets, dtype=np.int64)
    if len(off) != G + 1 or off[0] != 0 or off[-1] != M_total or np.any(np.diff(off) < 0):
        raise ValueError("bad group_offsets")
    N = B.shape[1]
    rows = np.arange(M_total) if rows is None else np.asarray(rows)
    cols = np.arange(N) if cols is None else np.asarray(cols)
    C = np.zeros((len(rows), len(cols)), np.float64)
    mass = np.zeros_like(C)
    for e in range(G):
        lo, hi = off[e], off[e + 1]
        sel = np.nonzero((rows >= lo) & (rows < hi))[0]
        if len(sel) == 0:
            continue
        local = rows[sel] - lo
        # the expert's A scale rows start at block lo / sa_rows; with one scale
        # per row a segment may start anywhere (packed segments)
        if lo % sa_rows:
            raise ValueError("with 128-row A scale blocks, segment starts must be multiples of 128")
        sA_e = sA[lo // sa_rows:(hi + sa_rows - 1) // sa_rows]
        Ce, me = gemm_blockscaled(A[lo:hi], sA_e, B[e], sB[e], rows=local, cols=cols,
                                  a_fmt=a_fmt, b_fmt=b_fmt, sa_rows=sa_rows)
        C[sel] = Ce
        mass[sel] = me
    return C, mass


def tolerance(C_ref: np.ndarray, mass: np.ndarray, out_dtype: str) -> np.ndarray:
    """Per-element bound on |C_gpu - C_ref| for an FP32-accumulating device.

    FP32 output: 1e-5 * mass + 1e-6.  BF16 output adds 2^-8 * |C_ref| for the
    final rounding to bfloat16.
    """
    bound = 1e-5 * mass + 1e-6
    if out_dtype == "bf16":
        bound = bound + 2.0 ** -8 * np.abs(C_ref)
    return bound
