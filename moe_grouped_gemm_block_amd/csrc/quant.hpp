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
// midpoint).  An approximate quotient y = a * fp32(1 / s_n), within a few
// ulp of a / s_n, only picks the two E4M3 grid values lo < hi around it (lo
// read off y's bits); the nearest grid value of the exact quotient is always
// one of them, because grid steps are at least 2^-4 of the value.  The
// choice is then exact: the midpoint m = (lo + hi) / 2 has at most 5
// significant bits, so fma(m, s_n, -a) has the sign of m s_n - a, i.e. of
// m - |x| / s, and is zero only at an exact tie, which goes to the even code.
// The scale fp32(double(amax) / 448) equals the IEEE FP32 quotient (double
// rounding through 53 bits is innocuous for one division of 24-bit numbers).
//
// Memory-bound: each element is read once (2 or 4 bytes) and written once
// (1 byte); about 20 FP32 / integer instructions per element.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
  float inv_n;  // fp32(1 / s_n), in (1, 2]
};

__device__ __forceinline__ ScaleNorm scale_norm(float s) {
  ScaleNorm n;
  n.e = __builtin_amdgcn_frexp_expf(s);
  n.s_n = __builtin_amdgcn_frexp_mantf(s);
  n.inv_n = 1.0f / n.s_n;
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
  const ScaleNorm sn = scale_norm(s);
  if (valid) {
    uint4* dst = reinterpret_cast<uint4*>(p.Q + e0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t packed = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) packed |= e4m3_code(v[16 * i + 4 * j + b], sn) << (8 * b);
        w[j] = packed;
      }
      dst[i] = uint4{w[0], w[1], w[2], w[3]};
    }
  }
  if (t == 0) p.S[size_t(rb) * Kb + kb] = s;
}

// 1 x 128 blocks.  Block b = row * Kb + kb covers elements [128 b, 128 b + 128)
// of the row-major matrix, so consecutive blocks are contiguous: a wave
// takes 4 of them (16 lanes each, 8 elements per lane: one 16-byte load of
// BF16, two of FP32), a workgroup 16.  amax is reduced within the 16 lanes.
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <bool IN_BF16>
__device__ __forceinline__ void quant1_body(const QuantArgs& p) {
  const long long nblk = (long long)p.M * (p.K / 128);
  const int lane = threadIdx.x & 63;
  const long long b = (long long)blockIdx.x * 16 + (threadIdx.x >> 6) * 4 + (lane >> 4);
  const bool valid = b < nblk;
  const size_t e0 = size_t(b) * 128 + size_t(lane & 15) * 8;   // first element of this lane
  float v[8];
  if (valid) {
    if constexpr (IN_BF16) {
      const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.X) + e0);
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_to_f32(u[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_to_f32(u[j] >> 16);
      }
    } else {
      const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(p.X) + e0);
      const float4 w0 = src[0], w1 = src[1];
      v[0] = w0.x; v[1] = w0.y; v[2] = w0.z; v[3] = w0.w;
      v[4] = w1.x; v[5] = w1.y; v[6] = w1.z; v[7] = w1.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;                    // joins the reduction, stores nothing
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(v[i]));
  amax = group16_max(amax);
  const float s = scale_of(amax);
  const ScaleNorm sn = scale_norm(s);
  if (valid) {
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) lo |= e4m3_code(v[i], sn) << (8 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) hi |= e4m3_code(v[4 + i], sn) << (8 * i);
    *reinterpret_cast<uint2*>(p.Q + e0) = uint2{lo, hi};
    if ((lane & 15) == 0) p.S[b] = s;
  }
}

#define DG_QUANT_KERNEL_DEF(NAME, BODY, BF16) \
  __global__ __launch_bounds__(256) void NAME(QuantArgs p) { BODY<BF16>(p); }
#define DG_QUANT_KERNEL_DECL(NAME, BODY, BF16) __global__ __launch_bounds__(256) void NAME(QuantArgs p);
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_128x128_bf16, quant128_body, true)
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_128x128_f32, quant128_body, false)
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_1x128_bf16, quant1_body, true)
DG_KERNEL(DG_QUANT_KERNEL, MISC)(dg_quant_1x128_f32, quant1_body, false)
#undef DG_QUANT_KERNEL_DECL
#undef DG_QUANT_KERNEL_DEF

}  // namespace dg
