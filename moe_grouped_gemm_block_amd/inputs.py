"""Seeded synthetic operands for the FP8 block-scaled GEMM workloads.

This module only *prepares inputs*: Gaussian data, per-block amax scaling and
round-to-nearest-even encoding to OCP E4M3FN bytes, plus MoE token routing.
It performs none of the GEMM's arithmetic (no decode, no products, no
accumulation), so both the HIP path and the CPU oracle can consume its output
without sharing any of the method's code.

Sources (the DeepGEMM pages this library follows):
  * Block-wise scaling, one FP32 factor per 128x128 block of A (M x K) and of
    B: DeepGEMM FP8-for-MoE page (2kiu.com/news/5461879), section 2.1; scales
    stored in FP32: same page, section 3.3.
  * E4M3 = 1 sign / 4 exponent / 3 mantissa bits, largest finite value 448:
    DeepGEMM FP8 kernel write-up (demingchina.com/news/60142), section 3.1
    table; FP8-for-MoE page section 2.1 (range about +-448).
  * Dynamic scaling (measure the range, map it onto the FP8 range): the
    low-precision essay (hotelren.com/news/5702847), section 2.1.
  * MoE contiguous layout (all experts' rows in one matrix, one launch): the
    shape-specialised-kernels page (nxmr.cn/news/132300), section 2.2.

Readings where the pages are silent (all fixed here, see the design notes):
  * scale s = fp32(amax / 448) per block, amax over |x| in fp32; an all-zero
    block gets s = 1 and all-zero codes.
  * code = RNE(x / s) with the quotient formed in float64 from fp32 x and s
    (so it is rounded only once), saturating at +-448 (E4M3FN has no inf);
    the NaN codes 0x7F / 0xFF are never produced; -0 (0x80) may appear.
  * B is stored N x K (K contiguous), its scales as [ceil(N/128)][K/128].
  * MoE: tokens ~ N(0,1); top-2 means two distinct experts; a token's row is
    copied into both experts' segments in token-id order; each segment is
    padded with zero rows to a multiple of 128; A is quantised over the padded
    contiguous layout.
  * Zipf(1.1) popularity: weight r^-1.1 for popularity rank r (ranks mapped to
    experts by a seeded permutation), top-2 drawn without replacement in
    proportion to weight, and the four lowest-ranked experts get weight 0 so
    that empty segments always occur.
  * numpy PCG64 streams: SeedSequence(seed).spawn(4) gives four independent
    streams for activations, weights, multipliers / outliers and routing, so
    that e.g. the routing of a workload does not depend on its weight sizes.
"""
from __future__ import annotations

import dataclasses

import numpy as np

BLOCK = 128
E4M3_MAX = 448.0
E5M2_MAX = 57344.0
FMT_MAX = {"e4m3": E4M3_MAX, "e5m2": E5M2_MAX}


# ---------------------------------------------------------------------------
# E4M3FN encoding (round to nearest, ties to even, saturating)
# ---------------------------------------------------------------------------

def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """float64 values -> uint8 OCP E4M3FN codes (RNE, saturate at +-448).

    Each |v| is snapped to the grid of its binade: quantum 2^(e-3) for a
    normal binade [2^e, 2^(e+1)), e >= -6, and 2^-9 below 2^-6 (the
    subnormals share the smallest normal binade's spacing).  Division by a
    power of two is exact, so ``np.rint`` (ties to even) performs the one and
    only rounding.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # binade exponent, subnormals -> -6
    quantum = np.ldexp(1.0, e - 3)
    r = np.minimum(np.rint(a / quantum) * quantum, E4M3_MAX)
    # r is now an exact E4M3 magnitude; split it into exponent / mantissa bits
    _, ex2 = np.frexp(r)
    e2 = ex2 - 1
    normal = r >= 2.0 ** -6
    exp_bits = np.where(normal, e2 + 7, 0).astype(np.int64)
    man = np.where(normal, r / np.ldexp(1.0, np.where(normal, e2, 0) - 3) - 8.0,
                   r * 512.0)
    code = (exp_bits << 3) | man.astype(np.int64)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


def encode_e5m2(v: np.ndarray) -> np.ndarray:
    """float64 values -> uint8 E5M2 codes (RNE, saturate at +-57344).

    Same binade snapping as encode_e4m3 with 2 mantissa bits and exponent
    bias 15: quantum 2^(e-2) in the binade [2^e, 2^(e+1)), e >= -14, and
    2^-16 below 2^-14.  An E5M2 code is the high byte of the IEEE half with
    the same value, which gives the bits directly.
    """
    v = np.asarray(v, dtype=np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E5M2_MAX)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -14)
    quantum = np.ldexp(1.0, e - 2)
    r = np.minimum(np.rint(a / quantum) * quantum, E5M2_MAX)    # exact half value with 2 mantissa bits
    code = (r.astype(np.float16).view(np.uint16) >> 8).astype(np.int64)
    code = code | (neg.astype(np.int64) << 7)
    return code.astype(np.uint8)


ENCODERS = {"e4m3": encode_e4m3, "e5m2": encode_e5m2}


def block_scales(x: np.ndarray, fmt: str = "e4m3", rows: int = BLOCK) -> np.ndarray:
    """Per-block scale fp32(amax/fmax) of a float32 [R][K] matrix (fmax = 448
    for E4M3, 57344 for E5M2), blocks of `rows` (128 or 1) x 128.

    Returns float32 [ceil(R/rows)][K/128]; all-zero blocks get 1.0.  The last
    row block may be partial (R not a multiple of rows).
    """
    R, K = x.shape
    assert rows in (1, BLOCK)
    Rb, Kb = -(-R // rows), -(-K // BLOCK)       # partial edge blocks in rows and in K
    xa = np.zeros((Rb * rows, Kb * BLOCK), np.float32)
    xa[:R, :K] = np.abs(x)
    amax = xa.reshape(Rb, rows, Kb, BLOCK).max(axis=(1, 3)).astype(np.float32)
    s = amax / np.float32(FMT_MAX[fmt])       # fp32 division, RNE
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    return s


def quantize(x: np.ndarray, row_chunk: int = 1024, fmt: str = "e4m3",
             rows: int = BLOCK) -> tuple[np.ndarray, np.ndarray]:
    """Quantise float32 [R][K] -> (codes uint8 [R][K], scales fp32 [ceil(R/rows)][K/128])
    with `rows` x 128 scale blocks (rows = 128 or 1)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    s = block_scales(x, fmt, rows)
    enc = ENCODERS[fmt]
    q = np.empty((R, K), np.uint8)
    s64 = s.astype(np.float64)
    for r0 in range(0, R, row_chunk):           # bounded temporaries
        r1 = min(R, r0 + row_chunk)
        srow = np.arange(r0, r1) // rows
        sexp = np.repeat(s64[srow], BLOCK, axis=1)[:, :K]   # [rows][K]
        q[r0:r1] = enc(x[r0:r1].astype(np.float64) / sexp)
    return q, s


# ---------------------------------------------------------------------------
# Problems
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Problem:
    """One GEMM workload: E4M3 codes, FP32 block scales and metadata.

    Dense: A [M][K], sA [ceil(M/sa_rows)][K/128], B [N][K], sB [ceil(N/128)][K/128].
    Grouped: A [M_total][K], B [G][N][K], sB [G][ceil(N/128)][K/128] and
    group_offsets int32 [G+1] (multiples of 128, o_0 = 0, o_G = M_total).
    """
    name: str
    A: np.ndarray
    sA: np.ndarray
    B: np.ndarray
    sB: np.ndarray
    M: int
    N: int
    K: int
    out_dtype: str                      # "f32" or "bf16"
    seed: int
    group_offsets: np.ndarray | None = None
    real_rows: int | None = None        # rows that carry tokens (grouped)
    a_fmt: str = "e4m3"                 # code format of A / B: "e4m3" or "e5m2"
    b_fmt: str = "e4m3"
    sa_rows: int = BLOCK                # rows per A scale block: 128 or 1 (per token)
    packed: bool = False                # grouped segments not padded to 128 rows
    group_counts: np.ndarray | None = None   # int32 [G]: real rows per expert (grouped)

    @property
    def grouped(self) -> bool:
        return self.group_offsets is not None

    @property
    def G(self) -> int:
        return 0 if self.group_offsets is None else len(self.group_offsets) - 1

    def algorithmic_flop(self) -> int:
        rows = self.real_rows if self.real_rows is not None else self.M
        return 2 * rows * self.N * self.K

    def padded_flop(self) -> int:
        return 2 * self.M * self.N * self.K

    def active_groups(self) -> int:
        """Experts with at least one row (all of them for a dense problem)."""
        if self.group_offsets is None:
            return 1
        return int(np.count_nonzero(np.diff(self.group_offsets)))

    def algorithmic_bytes(self) -> int:
        """A + sA + the B and sB of experts that have rows, read once; C written once."""
        cbytes = 4 if self.out_dtype == "f32" else 2
        G = max(self.G, 1)
        b = (self.B.nbytes + self.sB.nbytes) // G * self.active_groups()
        return (self.A.nbytes + self.sA.nbytes + b + self.M * self.N * cbytes
                + (0 if self.group_offsets is None else self.group_offsets.nbytes))


def streams(seed: int) -> list[np.random.Generator]:
    """Independent generators for activations, weights, modifiers, routing."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(4)]


def dense_problem(M: int, N: int, K: int, seed: int, out_dtype: str = "bf16",
                  a_std: float = 1.0, b_std: float = 1.0,
                  block_log2_range: float = 0.0, outlier_frac: float = 0.0,
                  outlier_mult: float = 50.0, name: str = "dense",
                  a_fmt: str = "e4m3", b_fmt: str = "e4m3", sa_rows: int = BLOCK) -> Problem:
    """Gaussian A [M][K] and B [N][K] with optional per-block multipliers and
    per-element outliers, quantised to E4M3 (or E5M2) with 128x128 block
    scales (A: sa_rows x 128 blocks)."""
    r_act, r_w, r_mod, _ = streams(seed)
    A = r_act.standard_normal((M, K), dtype=np.float32) * np.float32(a_std)
    B = r_w.standard_normal((N, K), dtype=np.float32) * np.float32(b_std)
    if block_log2_range:
        for X in (A, B):
            R = X.shape[0]
            Rb, Kb = -(-R // BLOCK), -(-K // BLOCK)
            u = r_mod.uniform(-block_log2_range, block_log2_range, size=(Rb, Kb))
            mult = np.exp2(u).astype(np.float32)
            full = np.repeat(np.repeat(mult, BLOCK, axis=0), BLOCK, axis=1)[:R, :K]
            X *= full
    if outlier_frac:
        hit = r_mod.random((M, K)) < outlier_frac
        A[hit] *= np.float32(outlier_mult)
    qA, sA = quantize(A, fmt=a_fmt, rows=sa_rows)
    qB, sB = quantize(B, fmt=b_fmt)
    return Problem(name=name, A=qA, sA=sA, B=qB, sB=sB, M=M, N=N, K=K,
                   out_dtype=out_dtype, seed=seed, a_fmt=a_fmt, b_fmt=b_fmt, sa_rows=sa_rows)


def route_top2(rng: np.random.Generator, T: int, weights: np.ndarray) -> np.ndarray:
    """Two distinct experts per token, drawn without replacement with
    probability proportional to ``weights`` (exponential-key method:
    key = log(u) / w, the two largest keys win).  Returns int [T][2]."""
    G = len(weights)
    u = rng.random((T, G))
    with np.errstate(divide="ignore"):
        keys = np.where(weights[None, :] > 0, np.log(u) / weights[None, :], -np.inf)
    top = np.argsort(-keys, axis=1, kind="stable")[:, :2]
    return top


def grouped_problem(G: int, N: int, K: int, T: int, seed: int,
                    popularity: str = "uniform", zipf_s: float = 1.1,
                    zero_lowest: int = 4, b_std: float = 0.02,
                    out_dtype: str = "bf16", name: str = "grouped", sa_rows: int = BLOCK) -> Problem:
    """MoE expert GEMM over the contiguous padded layout.

    Token activations X [T][K] ~ N(0,1); expert weights B_e [N][K] ~ N(0,b_std);
    every token goes to two distinct experts; expert e's segment holds its
    tokens' rows in token-id order, zero-padded to a multiple of 128 rows.
    """
    r_act, r_w, _, r_route = streams(seed)
    X = r_act.standard_normal((T, K), dtype=np.float32)
    Bq = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, -(-N // BLOCK), -(-K // BLOCK)), np.float32)
    for e in range(G):
        Be = r_w.standard_normal((N, K), dtype=np.float32) * np.float32(b_std)
        Bq[e], sB[e] = quantize(Be)
        del Be
    offsets, seg_tokens, counts = route(G, T, r_route, popularity, zipf_s, zero_lowest)
    M_total = int(offsets[-1])
    A = np.zeros((M_total, K), np.float32)
    for e in range(G):
        A[offsets[e]:offsets[e] + counts[e]] = X[seg_tokens[e]]
    qA, sA = quantize(A, rows=sa_rows)
    return Problem(name=name, A=qA, sA=sA, B=Bq, sB=sB, M=M_total, N=N, K=K,
                   out_dtype=out_dtype, seed=seed,
                   group_offsets=offsets.astype(np.int32),
                   real_rows=int(counts.sum()), sa_rows=sa_rows,
                   group_counts=np.asarray(counts, dtype=np.int32))


def route(G: int, T: int, rng: np.random.Generator, popularity: str = "uniform",
          zipf_s: float = 1.1, zero_lowest: int = 4, pad: int = BLOCK):
    """Top-2 routing of T tokens over G experts -> (offsets int64 [G+1],
    per-expert token ids, per-expert token counts).  Segments are padded to
    multiples of `pad` rows (1: packed)."""
    if popularity == "uniform":
        w = np.ones(G)
    elif popularity == "zipf":
        perm = rng.permutation(G)                 # perm[r-1] = expert of rank r
        w = np.zeros(G)
        ranks = np.arange(1, G + 1, dtype=np.float64)
        wr = ranks ** (-zipf_s)
        if zero_lowest:
            wr[G - zero_lowest:] = 0.0
        w[perm] = wr
    else:
        raise ValueError(popularity)
    top = route_top2(rng, T, w)
    counts = np.zeros(G, np.int64)
    seg_tokens = []
    for e in range(G):
        toks = np.nonzero((top == e).any(axis=1))[0]      # token-id order
        seg_tokens.append(toks)
        counts[e] = len(toks)
    padded = -(-counts // pad) * pad
    offsets = np.zeros(G + 1, np.int64)
    offsets[1:] = np.cumsum(padded)
    return offsets, seg_tokens, counts


def decode_problem(G: int, N: int, K: int, T: int, seed: int, popularity: str = "zipf",
                   zipf_s: float = 1.1, zero_lowest: int = 4, b_std: float = 0.02,
                   out_dtype: str = "bf16", name: str = "decode") -> Problem:
    """MoE expert GEMM of one decode step: T tokens, top-2 routing, packed
    segments (no padding rows) and one A scale per token and 128 columns.
    Same distributions as grouped_problem."""
    r_act, r_w, _, r_route = streams(seed)
    X = r_act.standard_normal((T, K), dtype=np.float32)
    Bq = np.empty((G, N, K), np.uint8)
    sB = np.empty((G, -(-N // BLOCK), -(-K // BLOCK)), np.float32)
    for e in range(G):
        Be = r_w.standard_normal((N, K), dtype=np.float32) * np.float32(b_std)
        Bq[e], sB[e] = quantize(Be)
        del Be
    offsets, seg_tokens, counts = route(G, T, r_route, popularity, zipf_s, zero_lowest, pad=1)
    A = np.concatenate([X[t] for t in seg_tokens], axis=0) if T else np.zeros((0, K), np.float32)
    qA, sA = quantize(A, rows=1)
    return Problem(name=name, A=qA, sA=sA, B=Bq, sB=sB, M=int(offsets[-1]), N=N, K=K,
                   out_dtype=out_dtype, seed=seed, group_offsets=offsets.astype(np.int32),
                   real_rows=int(counts.sum()), sa_rows=1, packed=True)


# ---------------------------------------------------------------------------
# The named workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "dense_256_f32",
    2: "dense_4096_blockmag_bf16",
    3: "skinny_m64_n12288_k4096_bf16",
    4: "moe_g8_n4096_k4096_uniform_bf16",
    5: "moe_g64_n2048_k2048_zipf_bf16",
    6: "moe_decode_g64_n2048_k2048_t128_zipf_bf16",
}


def make_config(i: int, seed: int | None = None, fmt: str = "e4m3", sa_rows: int = BLOCK) -> Problem:
    """Workload i (1..6); the default seed is the workload index.  Workload 6,
    a decode step of the MoE of workload 5 (128 tokens, packed segments,
    per-token A scales), always has sa_rows = 1.  fmt =
    "e5m2" quantises both operands of the dense workloads 1-3 to E5M2
    instead (same data, name suffixed with _e5m2).  sa_rows = 1 gives A one
    scale per token and 128 columns (name suffixed with _a1x128)."""
    s = i if seed is None else seed
    if fmt != "e4m3" and i > 3:
        raise ValueError("E5M2 variants exist for the dense workloads 1-3")
    sfx = ("" if fmt == "e4m3" else f"_{fmt}") + ("" if sa_rows == BLOCK else "_a1x128")
    kw = dict(a_fmt=fmt, b_fmt=fmt, sa_rows=sa_rows)
    if i == 1:
        return dense_problem(256, 256, 256, s, out_dtype="f32", name=CONFIG_NAMES[1] + sfx, **kw)
    if i == 2:
        return dense_problem(4096, 4096, 4096, s, out_dtype="bf16",
                             block_log2_range=4.0, name=CONFIG_NAMES[2] + sfx, **kw)
    if i == 3:
        return dense_problem(64, 12288, 4096, s, out_dtype="bf16", b_std=0.02,
                             outlier_frac=0.01, outlier_mult=50.0, name=CONFIG_NAMES[3] + sfx, **kw)
    if i == 4:
        return grouped_problem(8, 4096, 4096, 4096, s, popularity="uniform",
                               name=CONFIG_NAMES[4] + sfx, sa_rows=sa_rows)
    if i == 5:
        return grouped_problem(64, 2048, 2048, 8192, s, popularity="zipf",
                               name=CONFIG_NAMES[5] + sfx, sa_rows=sa_rows)
    if i == 6:
        return decode_problem(64, 2048, 2048, 128, s, popularity="zipf", name=CONFIG_NAMES[6])
    raise ValueError(f"unknown workload {i}")
