// Shared device helpers for the gfx950 FP8 block-scaled GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

typedef float v4f __attribute__((ext_vector_type(4)));

// Width of one K-block: the scale blocks are 128 x 128 (DeepGEMM FP8-for-MoE
// page, section 2.1), so every K-block's partial product is rescaled by one
// A and one B factor.
constexpr int KBLK = 128;

// LDS stages of the GEMM pipelines.  2 (the default): the next K-block's
// operands stream into one stage while the current one is read from the
// other.  1 (build with -DDG_STAGES=1, a debugging aid): every pipeline waits
// until the current K-block has been used before it loads the next one into
// the same stage.  The arithmetic and its order are the same, so both builds
// give identical bits; a difference points at a race between the loads into
// one stage and the reads of another (the "drop to a single buffer" check of
// the DeepGEMM FP8 kernel write-up, section 6.2).
#ifndef DG_STAGES
#define DG_STAGES 2
#endif
static_assert(DG_STAGES == 1 || DG_STAGES == 2, "DG_STAGES is 1 or 2");
constexpr bool kSingleStage = DG_STAGES == 1;

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

typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));

// 16 bytes to global memory, optionally as a non-temporal store (NT).  A
// kernel whose workgroups all write their tiles of C at the same moment, at
// the end of a single round, measured faster with non-temporal stores
// (4096^3 BF16: 0.1014-0.1021 vs 0.1039-0.1043 ms; M = 64 N = 12288:
// 15.5 vs 16.2 us); grouped and packed-segment kernels, whose stores overlap
// other workgroups' work, were ~1 % slower with them and keep plain stores.
template <bool NT>
__device__ __forceinline__ void store16(void* dst, u32x4_nt w) {
  if constexpr (NT) __builtin_nontemporal_store(w, static_cast<u32x4_nt*>(dst));
  else *static_cast<u32x4_nt*>(dst) = w;
}

// 16 bytes from global memory with a non-temporal load (data read once).
__device__ __forceinline__ uint4 load16_nt(const void* src) {
  const u32x4_nt w = __builtin_nontemporal_load(static_cast<const u32x4_nt*>(src));
  return uint4{w.x, w.y, w.z, w.w};
}

// Store the W consecutive output values v[0 .. W) of one row at columns
// n0 .. n0 + W - 1 of C (row-major, N columns; `row_off` = row * N elements),
// skipping columns >= N.  When every row starts 16-byte aligned (N % 8 == 0
// for BF16, N % 4 == 0 for FP32) whole 16-byte vectors are stored (NT: as
// non-temporal stores); otherwise element by element (a uniform branch on N).
template <bool OUT_BF16, int W, bool NT = false>
__device__ __forceinline__ void store_row_span(void* C, size_t row_off, int n0, int N, const float* v) {
  constexpr int VEC = OUT_BF16 ? 8 : 4;             // elements per 16 bytes
  static_assert(W % VEC == 0, "span of whole vectors");
  if (N % VEC == 0) {
#pragma unroll
    for (int c = 0; c < W / VEC; ++c) {
      const int n = n0 + VEC * c;
      if (n >= N) continue;                           // whole vector in or out
      if constexpr (OUT_BF16) {
        const u32x4_nt w = {pack_bf16x2(v[8 * c + 0], v[8 * c + 1]), pack_bf16x2(v[8 * c + 2], v[8 * c + 3]),
                            pack_bf16x2(v[8 * c + 4], v[8 * c + 5]), pack_bf16x2(v[8 * c + 6], v[8 * c + 7])};
        store16<NT>(static_cast<uint16_t*>(C) + row_off + n, w);
      } else {
        const u32x4_nt w = {__builtin_bit_cast(uint32_t, v[4 * c]), __builtin_bit_cast(uint32_t, v[4 * c + 1]),
                            __builtin_bit_cast(uint32_t, v[4 * c + 2]), __builtin_bit_cast(uint32_t, v[4 * c + 3])};
        store16<NT>(static_cast<float*>(C) + row_off + n, w);
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
