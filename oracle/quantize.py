"""CPU oracle for FP8 (E4M3) block quantisation of activations -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this module.  The product path never imports it, and it imports nothing from
the product path or from the input generator.

What it computes, per block of R rows x 128 columns (R = 128: the 128 x 128
blocks of the GEMM operands; R = 1: one scale per token and 128-column group):

    amax = max |x| over the block          (x in FP32)
    s    = fp32(amax / 448)                (1 for an all-zero block)
    q    = the E4M3FN code whose value is nearest to x / s, the quotient taken
           in float64; ties go to the code with an even last bit (i.e. an even
           mantissa); magnitudes at or above 448 give 448 (E4M3FN has no
           infinity, and the NaN codes are never produced); the sign bit is
           the sign bit of x, so -0 is kept.

Sources:
  * Block-wise scaling with one factor per block, e.g. 128 x 128:
    DeepGEMM FP8-for-MoE page (2kiu.com/news/5461879), section 2.1; FP32
    scale factors: same page, section 3.3; activations re-scaled on the fly
    during inference: same page, section 4.3.
  * Dynamic (amax) scaling that maps the measured range onto the FP8 range:
    the low-precision essay (hotelren.com/news/5702847), section 2.1.
  * Per-group scaling along K with groups of 128 (the 1 x 128 case):
    DeepGEMM FP8 kernel write-up (demingchina.com/news/60142), section 5.2.
  * E4M3 layout and its largest finite value 448: the same write-up,
    section 3.1 table.
Readings where the pages are silent (the amax/448 map, RNE, float64
quotient, saturation, scale 1 for all-zero blocks) are the ones the operand
generator of this repository also follows.

The encoder here is deliberately not the binade arithmetic a kernel would
use: it searches the sorted table of the 127 finite non-negative E4M3 values
for the two neighbours of |x / s| and compares distances, so that it can be
checked by eye against the definition.
"""
from __future__ import annotations

import numpy as np

from .blockscaled import decode_table

E4M3_MAX = 448.0

# Non-negative finite E4M3 values, codes 0x00 .. 0x7E, strictly increasing.
_POS_VALUES = decode_table()[:0x7F].copy()
assert np.all(np.diff(_POS_VALUES) > 0) and _POS_VALUES[-1] == E4M3_MAX


def encode_nearest(v: np.ndarray) -> np.ndarray:
    """float64 -> E4M3FN codes: nearest value, ties to the even code, capped
    at 448, sign bit taken from v."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    hi = np.searchsorted(_POS_VALUES, a, side="left")      # first value >= a
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= E4M3_MAX, 0x7E, code)            # saturate
    code = np.where(a <= _POS_VALUES[0], 0, code)          # a == 0
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def quantize_blockscaled(x: np.ndarray, block_rows: int) -> tuple[np.ndarray, np.ndarray]:
    """float32 [M][K] -> (codes uint8 [M][K], scales float32 [ceil(M/R)][K/128])."""
    if block_rows not in (1, 128):
        raise ValueError("block_rows must be 1 or 128")
    x = np.asarray(x, dtype=np.float32)
    M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    R, Kb = block_rows, K // 128
    Rb = -(-M // R)
    q = np.empty((M, K), np.uint8)
    s = np.empty((Rb, Kb), np.float32)
    for rb in range(Rb):
        r0, r1 = rb * R, min(M, rb * R + R)
        for kb in range(Kb):
            blk = x[r0:r1, kb * 128:(kb + 1) * 128]
            amax = float(np.max(np.abs(blk)))                      # exact, fp32 values
            sc = np.float32(1.0) if amax == 0.0 else np.float32(amax / E4M3_MAX)
            s[rb, kb] = sc
            q[r0:r1, kb * 128:(kb + 1) * 128] = encode_nearest(blk.astype(np.float64) / np.float64(sc))
    return q, s
