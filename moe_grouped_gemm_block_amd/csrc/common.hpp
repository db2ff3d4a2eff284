// Shared device helpers for the gfx950 FP8 block-scaled GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Width of one K-block: the scale blocks are 128 x 128 (DeepGEMM FP8-for-MoE
// page, section 2.1), and one 16x16x128 FP8 MFMA consumes exactly one K-block.
constexpr int KBLK = 128;

// 16x16 output tile, K = 128 FP8 E4M3 products per element, FP32 result,
// no input accumulator.  Zero E8M0 scale operands select the unscaled
// v_mfma_f32_16x16x128_f8f6f4 encoding; format code 0 = FP8 E4M3 for both
// operands.
//
// Register layout (identical for both operands): lane l supplies row / column
// (l % 16) and the 32 consecutive K bytes [32 (l / 16), 32 (l / 16) + 32).
// Output: lane l holds D[4 (l / 16) + r][l % 16], r = 0..3, where the first
// index runs over `a`'s rows and the second over `b`'s rows.
__device__ __forceinline__ v4f mfma16_fp8(const v8i& a, const v8i& b) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, zero, 0, 0, 0, 0, 0, 0);
}

// Same instruction, accumulating into `c`.
__device__ __forceinline__ v4f mfma16_fp8_acc(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// FP32 -> BF16, round to nearest even (NaN stays NaN): gfx950 converts two
// values per instruction (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

__device__ __forceinline__ uint32_t bf16_bits(float f) { return pack_bf16x2(f, 0.f) & 0xFFFFu; }

// Buffer offset that lies past any buffer's end (num_records <= 2^31 here):
// a load from it returns zeros.  Row offsets below 2^31 can be added to it
// without wrapping.
constexpr uint32_t kOutOfRange = 0x80000000u;

// Store the W consecutive output values v[0 .. W) of one row at columns
// n0 .. n0 + W - 1 of C (row-major, N columns; `row_off` = row * N elements),
// skipping columns >= N.  When every row starts 16-byte aligned (N % 8 == 0
// for BF16, N % 4 == 0 for FP32) whole 16-byte vectors are stored; otherwise
// element by element (a uniform branch on N).
template <bool OUT_BF16, int W>
__device__ __forceinline__ void store_row_span(void* C, size_t row_off, int n0, int N, const float* v) {
  constexpr int VEC = OUT_BF16 ? 8 : 4;             // elements per 16 bytes
  static_assert(W % VEC == 0, "span of whole vectors");
  if (N % VEC == 0) {
#pragma unroll
    for (int c = 0; c < W / VEC; ++c) {
      const int n = n0 + VEC * c;
      if (n >= N) continue;                           // whole vector in or out
      if constexpr (OUT_BF16) {
        uint4 w;
        w.x = pack_bf16x2(v[8 * c + 0], v[8 * c + 1]);
        w.y = pack_bf16x2(v[8 * c + 2], v[8 * c + 3]);
        w.z = pack_bf16x2(v[8 * c + 4], v[8 * c + 5]);
        w.w = pack_bf16x2(v[8 * c + 6], v[8 * c + 7]);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(C) + row_off + n) = w;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(C) + row_off + n) =
            float4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < W; ++t) {
      const int n = n0 + t;
      if (n >= N) continue;
      if constexpr (OUT_BF16)
        static_cast<uint16_t*>(C)[row_off + n] = uint16_t(bf16_bits(v[t]));
      else
        static_cast<float*>(C)[row_off + n] = v[t];
    }
  }
}

// 16-byte granule swizzle inside a 128-byte LDS row: row r's granule g is
// stored at slot g ^ ((r ^ (r >> 3)) & 7).  Eight consecutive rows, and the
// two 8-row halves of sixteen consecutive rows, then hit distinct slots, so
// the per-lane 16-byte reads of an MFMA fragment (16 rows, same granule) are
// spread over all banks instead of piling onto one 16-byte column.  This is
// the XOR row swizzle of the DeepGEMM FP8 kernel write-up (section 4.2),
// re-derived for 16-byte granules.
__device__ __forceinline__ int swz(int r, int g) { return g ^ ((r ^ (r >> 3)) & 7); }

// Grouped GEMM: the expert owning row m0, i.e. the last e with
// offs[e] <= m0 (empty experts are skipped automatically).  Returns G when
// m0 lies past the last segment.
__device__ __forceinline__ int find_group(const int32_t* __restrict__ offs, int G, int m0) {
  int lo = 0, hi = G;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offs[mid] <= m0) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace dg
