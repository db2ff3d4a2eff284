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
// Exactness.  The quotient is the correctly rounded double x / s.  An E4M3
// midpoint m has at most 5 significant bits, so m s is exact in 29 bits.  If
// x = m s the double quotient is exactly m (a tie, resolved to even); if not,
// x and m s are distinct multiples of a unit at most 2^-29 |m s|, so
// |x / s - m| is far above the double's 2^-53 relative rounding error and
// rounding the double gives the same code as rounding the exact quotient.
// The scale fp32(double(amax) / 448) equals the IEEE FP32 quotient (double
// rounding through 53 bits is innocuous for one division of 24-bit numbers).
//
// Memory-bound: each element is read once (2 or 4 bytes) and written once
// (1 byte); the per-element double division is a few percent of the issue
// slots at this traffic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

struct QuantArgs {
  const void* X;          // [M][K] FP32 or BF16
  uint8_t* Q;             // [M][K] E4M3FN codes
  float* S;               // [ceil(M/R)][K/128]
  int M, K;
};

// double -> E4M3FN code: nearest value, ties to even, capped at 448.
__device__ __forceinline__ uint32_t e4m3_rne(double q) {
  const uint32_t sign = uint32_t(uint64_t(__double_as_longlong(q)) >> 63) << 7;   // 0 or 0x80
  const double a = __builtin_fabs(q);
  if (!(a < 448.0)) return sign | 0x7Eu;                  // saturate (also NaN: unspecified input)
  if (a < 0.015625) {                                     // below 2^-6: steps of 2^-9
    return sign | uint32_t(__builtin_rint(a * 512.0));    // 0 .. 8 (8 = 2^-6, code 0x08)
  }
  // a in [2^E, 2^(E+1)), -6 <= E <= 8: 8 steps of 2^(E-3) per binade
  const int E = int((__double_as_longlong(a) >> 52) & 0x7FF) - 1023;
  const double to_steps = __longlong_as_double((long long)(1023 + 3 - E) << 52);   // 2^(3-E), exact
  uint32_t m = uint32_t(__builtin_rint(a * to_steps));    // 8 .. 16 (16: carried into the next binade)
  uint32_t e = uint32_t(E + 7);
  if (m == 16) { m = 8; e += 1; }                         // a < 448 keeps this below 448
  return sign | (e << 3) | (m - 8);
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

// 128 x 128 blocks: one workgroup of 256 threads per block, block index
// rb * Kb + kb; thread t holds row t/2, columns 64 (t%2) .. 64 (t%2) + 63.
template <bool IN_BF16>
__device__ __forceinline__ void quant128_body(const QuantArgs& p) {
  const int Kb = p.K / 128;
  const int rb = blockIdx.x / Kb, kb = blockIdx.x % Kb;
  const int t = threadIdx.x, r = t >> 1, h = t & 1;
  const int m = rb * 128 + r;
  const bool valid = m < p.M;
  const size_t e0 = size_t(m) * p.K + size_t(kb) * 128 + 64 * h;   // first element of this thread
  float v[64];
  if (valid) {
    if constexpr (IN_BF16) {
      const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.X) + e0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint4 w = src[i];
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[8 * i + 2 * j] = bf16_to_f32(u[j] & 0xFFFFu);
          v[8 * i + 2 * j + 1] = bf16_to_f32(u[j] >> 16);
        }
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.X) + e0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float4 w = src[i];
        v[4 * i] = w.x; v[4 * i + 1] = w.y; v[4 * i + 2] = w.z; v[4 * i + 3] = w.w;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) v[i] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
  amax = wave_max(amax);
  __shared__ float wmax[4];
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = scale_of(amax);
  const double sd = double(s);
  if (valid) {
    uint4* dst = reinterpret_cast<uint4*>(p.Q + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) packed |= e4m3_rne(double(v[16 * i + 4 * j + b]) / sd) << (8 * b);
        w[j] = packed;
      }
      dst[i] = uint4{w[0], w[1], w[2], w[3]};
    }
  }
  if (t == 0) p.S[size_t(rb) * Kb + kb] = s;
}

// 1 x 128 blocks: one wave per (row, 128-column group), block index
// row * Kb + kb = 4 * workgroup + wave; lane L holds columns 2L, 2L + 1.
template <bool IN_BF16>
__device__ __forceinline__ void quant1_body(const QuantArgs& p) {
  const int Kb = p.K / 128;
  const int lane = threadIdx.x & 63;
  const long long blk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= (long long)p.M * Kb) return;       // whole wave; no barrier in this kernel
  const int m = int(blk / Kb), kb = int(blk % Kb);
  const size_t e0 = size_t(m) * p.K + size_t(kb) * 128 + 2 * lane;
  float v0, v1;
  if constexpr (IN_BF16) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(p.X) + e0);
    v0 = bf16_to_f32(w & 0xFFFFu);
    v1 = bf16_to_f32(w >> 16);
  } else {
    const float2 w = *reinterpret_cast<const float2*>(static_cast<const float*>(p.X) + e0);
    v0 = w.x; v1 = w.y;
  }
  const float amax = wave_max(fmaxf(__builtin_fabsf(v0), __builtin_fabsf(v1)));
  const float s = scale_of(amax);
  const double sd = double(s);
  const uint32_t c = e4m3_rne(double(v0) / sd) | (e4m3_rne(double(v1) / sd) << 8);
  *reinterpret_cast<uint16_t*>(p.Q + e0) = uint16_t(c);
  if (lane == 0) p.S[size_t(m) * Kb + kb] = s;
}

#define DG_QUANT_KERNEL(NAME, BODY, BF16) \
  __global__ __launch_bounds__(256) void NAME(QuantArgs p) { BODY<BF16>(p); }
DG_QUANT_KERNEL(dg_quant_128x128_bf16, quant128_body, true)
DG_QUANT_KERNEL(dg_quant_128x128_f32, quant128_body, false)
DG_QUANT_KERNEL(dg_quant_1x128_bf16, quant1_body, true)
DG_QUANT_KERNEL(dg_quant_1x128_f32, quant1_body, false)
#undef DG_QUANT_KERNEL

}  // namespace dg
