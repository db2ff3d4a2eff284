// FP8 (E4M3FN) block quantisation of activations, gfx950: the step that
// produces the A operand of the block-scaled GEMM and its scales.
//
// Per block of R rows x 128 columns (R = 128: the GEMM's 128 x 128 operand
// blocks; R = 1: one scale per token and 128-column group):
//   amax = max |x|;  s = fp32(amax / 448), 1 for an all-zero block;
//   q = x / s rounded to the nearest E4M3FN value (ties to even), capped at
//   +-448, sign bit from x.
// Block-wise scaling: DeepGEMM FP8-for-MoE page (2kiu.com/news/5461879),
// section 2.1, activations re-scaled on the fly at inference: section 4.3;
// amax-based dynamic scaling: low-precision essay (hotelren.com/news/5702847),
// section 2.1; 1 x 128 groups along K: DeepGEMM FP8 kernel write-up
// (demingchina.com/news/60142), section 5.2; E4M3 range: same write-up,
// section 3.1.
//
// Exactness without a per-element division.  Per block the scale is brought
// to s_n = s 2^-e in [0.5, 1) by its binary exponent e (exact, subnormal s
// included) and each |x| to a = |x| 2^-e (exact: a <= |x| / s * s_n < 448 can
// not overflow, and an a that underflows is far below the first E4M3
// midpoint).  An approximate quotient y = a * inv_n (inv_n = 1 / s_n within
// one ulp), within a few ulp of a / s_n, only picks the two E4M3 grid values lo < hi around it (lo
// read off y's bits); the nearest grid value of the exact quotient is always
// one of them, because grid steps are at least 2^-4 of the value.  The
// choice is then exact: the midpoint m = (lo + hi) / 2 has at most 5
// significant bits, so fma(m, s_n, -a) has the sign of m s_n - a, i.e. of
// m - |x| / s, and is zero only at an exact tie, which goes to the even code.
// The scale fp32(double(amax) / 448) equals the IEEE FP32 quotient (double
// rounding through 53 bits is innocuous for one division of 24-bit numbers).
//
// Memory-bound: each element is read once (2 or 4 bytes) and written once
// (1 byte), both with non-temporal loads and stores (4096 x 4096 BF16, 1 x 128
// blocks: 15.3 -> 14.0 us; 128 x 128: 16.9 -> 16.4 us).  The encoder above
// takes about 20 instructions per element; the kernels use it only as the
// fallback of a cheaper one (fast_codes4 below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"
#include "kernels.hpp"

namespace dg {

struct QuantArgs {
  const void* X;          // [M][K] FP32 or BF16
  uint8_t* Q;             // [M][K] E4M3FN codes
  float* S;               // [ceil(M/R)][K/128]
  int M, K;
};

// Per-block constants of the exact encoder (see "Exactness" above).
struct ScaleNorm {
  int e;        // s = s_n 2^e
  float s_n;    // in [0.5, 1)
  float inv_n;  // 1 / s_n within one ulp, in (1, 2]
};

__device__ __forceinline__ ScaleNorm scale_norm(float s) {
  ScaleNorm n;
  n.e = __builtin_amdgcn_frexp_expf(s);
  n.s_n = __builtin_amdgcn_frexp_mantf(s);
  // only an approximation is needed (the decisions below are exact): the
  // hardware reciprocal, within one ulp
  n.inv_n = __builtin_amdgcn_rcpf(n.s_n);
  return n;
}

// E4M3FN code of x / s: nearest value, ties to even, capped at 448, sign of x.
__device__ __forceinline__ uint32_t e4m3_code(float x, const ScaleNorm& n) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = __builtin_ldexpf(__builtin_fabsf(x), -n.e);
  const float y = a * n.inv_n;                            // ~ |x| / s
  // Grid point at or below y, read off the FP32 bits: in [2^E, 2^(E+1))
  // (E >= -6) the E4M3 code is ((E + 7) << 3) | m for the top three mantissa
  // bits m, i.e. (bits >> 20) - (120 << 3).  Below 2^-6 the grid (codes
  // 0 .. 8, spacing 2^-9) is that of [2^-6, 2^-5) shifted down by 2^-6, so y
  // is moved there first; that addition may round, but only across a grid
  // point that y is within an ulp of, where the decision below still picks
  // the nearest value.
  const bool sub = y < 0x1p-6f;
  const float c = sub ? 0x1p-6f : 0.f;
  const uint32_t tb = __float_as_uint(y + c);
  const uint32_t lo = (tb >> 20) - (sub ? 968u : 960u);
  // midpoint above that grid point: one more mantissa bit (exact, 5
  // significant bits), moved back by c (exact)
  const float mid = __uint_as_float((tb & 0xFFF00000u) | 0x00080000u) - c;
  const float r = __builtin_fmaf(mid, n.s_n, -a);         // sign of mid - |x|/s, exact
  const uint32_t up = uint32_t(r < 0.f || (r == 0.f && (lo & 1u)));   // nearest, ties to even
  // a code past 0x7E (above 448, or the carry into the next binade at the
  // top) saturates
  return sign | min(lo + up, 0x7Eu);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float scale_of(float amax) {
  return amax > 0.f ? float(double(amax) / 448.0) : 1.0f;
}

// BF16 bits -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// ---- fast encoder -----------------------------------------------------------
// Per block, r = fp32(1 / s_n) 2^-e, so x r is x / s up to three FP32
// roundings.  With r_lo = fp32(r (1 - 2^-20)) and r_hi = fp32(r (1 + 2^-20)),
// y_lo = fp32(x r_lo) and y_hi = fp32(x r_hi) bracket the exact quotient x / s
// (each rounding moves a value by at most 2^-24 of it).  The hardware
// conversion (v_cvt_scalef32_pk_fp8_f32, scale 1: round to nearest even in
// OCP E4M3) is monotone, so when it gives the same code for y_lo and y_hi that
// is also the code of x / s.  The codes differ only when a midpoint of the E4M3
// grid lies within about 2^-20 of x / s (or at the top of the range, where
// y_hi may exceed 448 and convert to NaN): those lanes, and every element of a
// block whose r is not a normal FP32 number (scales near the ends of the FP32
// range), are encoded by the exact encoder e4m3_code instead.  Zero, -0,
// subnormal E4M3 codes and saturation need no separate treatment.
struct FastScale {
  float r_lo, r_hi;
  bool ok;      // r is a normal FP32 number
};

__device__ __forceinline__ FastScale fast_scale(const ScaleNorm& n) {
  const float r = __builtin_ldexpf(n.inv_n, -n.e);
  FastScale f;
  f.r_lo = r * (1.0f - 0x1p-20f);
  f.r_hi = r * (1.0f + 0x1p-20f);
  f.ok = __builtin_fabsf(r) >= 0x1p-125f && __builtin_fabsf(r) <= 0x1p+126f;
  return f;
}

typedef short v2i16 __attribute__((ext_vector_type(2)));

// Codes of y0..y3 (value i in byte i) by the hardware conversion.
__device__ __forceinline__ uint32_t hw_codes4(float y0, float y1, float y2, float y3) {
  v2i16 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(v2i16{0, 0}, y0, y1, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, y2, y3, 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
}

// Four values -> four E4M3 codes (value i in byte i); `miss` is raised when
// the bracket does not decide one of them.
__device__ __forceinline__ uint32_t fast_codes4(float x0, float x1, float x2, float x3, const FastScale& f,
                                                bool& miss) {
  const uint32_t lo = hw_codes4(x0 * f.r_lo, x1 * f.r_lo, x2 * f.r_lo, x3 * f.r_lo);
  const uint32_t hi = hw_codes4(x0 * f.r_hi, x1 * f.r_hi, x2 * f.r_hi, x3 * f.r_hi);
  miss = miss | (lo != hi);
  return lo;
}

__device__ __forceinline__ uint32_t exact_codes4(float x0, float x1, float x2, float x3, const ScaleNorm& sn) {
  return e4m3_code(x0, sn) | (e4m3_code(x1, sn) << 8) | (e4m3_code(x2, sn) << 16) | (e4m3_code(x3, sn) << 24);
}

// ---- 1 x 128 blocks ----------------------------------------------------------
// Block b = row * Kb + kb covers elements [128 b, 128 b + 128) of the
// row-major matrix, so consecutive blocks are contiguous.  An 8-lane group
// takes one block (16 elements per lane: two 16-byte loads of BF16, four of
// FP32), a wave 8 consecutive blocks, a workgroup 32.  amax is reduced within
// the 8 lanes by DPP lane permutations.
__device__ __forceinline__ float group8_max(float v) {
  // lane i of each 8-lane group takes the max with lane 7 - i (half-row
  // mirror), then with lane 3 - i of its quad, then with lane i ^ 1: after
  // the three steps every lane holds the max of its 8 lanes
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     0x141, 0xF, 0xF, false)));   // row_half_mirror
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     0x1B, 0xF, 0xF, false)));    // quad_perm 3,2,1,0
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                                     0xB1, 0xF, 0xF, false)));    // quad_perm 1,0,3,2
  return v;
}

template <bool IN_BF16>
struct Q1Buf {
  uint4 w[IN_BF16 ? 2 : 4];
};

template <bool IN_BF16>
__device__ __forceinline__ float q1_value(const Q1Buf<IN_BF16>& b, int i) {
  if constexpr (IN_BF16) {
    const uint4 w = b.w[i / 8];
    const uint32_t u = (i % 8) < 2 ? w.x : (i % 8) < 4 ? w.y : (i % 8) < 6 ? w.z : w.w;
    return (i & 1) ? __uint_as_float(u & 0xFFFF0000u) : bf16_to_f32(u & 0xFFFFu);
  } else {
    const uint4 w = b.w[i / 4];
    return __uint_as_float((i % 4) == 0 ? w.x : (i % 4) == 1 ? w.y : (i % 4) == 2 ? w.z : w.w);
  }
}

template <bool IN_BF16>
__device__ __forceinline__ void q1_load(Q1Buf<IN_BF16>& b, const QuantArgs& p, long long blk, long long nblk) {
  const int lane = threadIdx.x & 63;
  constexpr int N = IN_BF16 ? 2 : 4;
  if (blk < nblk) {
    const size_t e0 = size_t(blk) * 128 + size_t(lane & 7) * 16;
    const uint4* src = IN_BF16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.X) + e0)
                               : reinterpret_cast<const uint4*>(static_cast<const float*>(p.X) + e0);
#pragma unroll
    for (int i = 0; i < N; ++i) b.w[i] = load16_nt(src + i);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) b.w[i] = uint4{0u, 0u, 0u, 0u};   // joins the reduction
  }
}

template <bool IN_BF16>
__device__ __forceinline__ void q1_process(const Q1Buf<IN_BF16>& b, const QuantArgs& p, long long blk,
                                           long long nblk) {
  const int lane = threadIdx.x & 63;
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(q1_value(b, i)));
  amax = group8_max(amax);
  const float s = scale_of(amax);
  const ScaleNorm sn = scale_norm(s);
  const FastScale fs = fast_scale(sn);
  if (blk < nblk) {
    bool flag = !fs.ok;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = fast_codes4(q1_value(b, 4 * j), q1_value(b, 4 * j + 1), q1_value(b, 4 * j + 2),
                         q1_value(b, 4 * j + 3), fs, flag);
    if (flag) {                                   // rare: redo this lane's codes exactly
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = exact_codes4(q1_value(b, 4 * j), q1_value(b, 4 * j + 1), q1_value(b, 4 * j + 2),
                            q1_value(b, 4 * j + 3), sn);
    }
    store16<true>(p.Q + size_t(blk) * 128 + size_t(lane & 7) * 16, u32x4_nt{w[0], w[1], w[2], w[3]});
    if ((lane & 7) == 0) p.S[blk] = s;
  }
}

template <bool IN_BF16>
__device__ __forceinline__ void quant1_body(const QuantArgs& p) {
  const long long nblk = (long long)p.M * (p.K / 128);
  const long long blk = (long long)blockIdx.x * 32 + (threadIdx.x >> 3);   // 32 blocks per workgroup
  Q1Buf<IN_BF16> b;
  q1_load(b, p, blk, nblk);
  q1_process(b, p, blk, nblk);
}

// ---- 128 x 128 blocks --------------------------------------------------------
// One workgroup of 1024 threads per block (block index rb * Kb + kb); thread
// t holds row t / 8, columns 16 (t % 8) .. 16 (t % 8) + 15 of the block, so a
// wave reads 8 whole rows (whole 128-byte lines) and writes 8 whole rows of
// codes.  The block amax goes through a wave reduction and 16 per-wave
// maxima in LDS.  (Four threads per row with 32 values each, or a persistent
// workgroup that loaded the next block while encoding the current one, were
// slower: fewer waves in flight.)
template <bool IN_BF16>
__device__ __forceinline__ void quant128_body(const QuantArgs& p) {
  __shared__ float wmax[16];
  const int Kb = p.K / 128;
  const int rb = blockIdx.x / Kb, kb = blockIdx.x - rb * Kb;
  const int t = threadIdx.x;
  const int m = rb * 128 + (t >> 3);
  const size_t e0 = size_t(m) * p.K + size_t(kb) * 128 + 16 * (t & 7);
  // the same 16-value layout as the 1 x 128 kernel (Q1Buf); rows past M read 0
  Q1Buf<IN_BF16> b;
  constexpr int N = IN_BF16 ? 2 : 4;
  if (m < p.M) {
    const uint4* src = IN_BF16 ? reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.X) + e0)
                               : reinterpret_cast<const uint4*>(static_cast<const float*>(p.X) + e0);
#pragma unroll
    for (int i = 0; i < N; ++i) b.w[i] = load16_nt(src + i);
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) b.w[i] = uint4{0u, 0u, 0u, 0u};
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, __builtin_fabsf(q1_value(b, i)));
  amax = wave_max(amax);
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = wmax[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) amax = fmaxf(amax, wmax[w]);
  const float s = scale_of(amax);
  const ScaleNorm sn = scale_norm(s);
  const FastScale fs = fast_scale(sn);
  if (m < p.M) {
    bool flag = !fs.ok;
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = fast_codes4(q1_value(b, 4 * j), q1_value(b, 4 * j + 1), q1_value(b, 4 * j + 2),
                         q1_value(b, 4 * j + 3), fs, flag);
    if (flag) {                                   // rare: redo this thread's codes exactly
#pragma unroll
      for (int j = 0; j < 4; ++j)
        w[j] = exact_codes4(q1_value(b, 4 * j), q1_value(b, 4 * j + 1), q1_value(b, 4 * j + 2),
                            q1_value(b, 4 * j + 3), sn);
    }
    store16<true>(p.Q + e0, u32x4_nt{w[0], w[1], w[2], w[3]});
  }
  if (t == 0) p.S[size_t(rb) * Kb + kb] = s;
}

#define DG_QUANT_KERNEL_DEF(NAME, BODY, BF16, THREADS) \
  __global__ __launch_bounds__(THREADS) void NAME(QuantArgs p) { BODY<BF16>(p); }
#define DG_QUANT_KERNEL_DECL(NAME, BODY, BF16, THREADS) __global__ __launch_bounds__(THREADS) void NAME(QuantArgs p);
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_128x128_bf16, quant128_body, true, 1024)
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_128x128_f32, quant128_body, false, 1024)
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_1x128_bf16, quant1_body, true, 256)
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_1x128_f32, quant1_body, false, 256)
#undef DG_QUANT_KERNEL_DECL
#undef DG_QUANT_KERNEL_DEF

}  // namespace dg
