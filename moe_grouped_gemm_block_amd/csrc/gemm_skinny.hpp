// Block-scaled FP8 GEMM for few rows (M <= 64, decode-style shapes), gfx950.
//
// Same arithmetic as the tiled kernel (exact FP8 -> FP16 conversion, FP16
// MFMA partial per 128-wide K-block, FP32 rescale by fp32(sA * sB), FP32
// accumulation; DeepGEMM FP8-for-MoE page, 2kiu.com/news/5461879, sections 2.1
// and 3.3), organised for a shape whose cost is streaming B once from HBM:
// with M = 64, every byte of B feeds only 128 FLOP.
//
//   * one workgroup per 16*NI columns of C (all rows); its 4 waves split the
//     K-blocks (wave w takes kb = w, w+4, ...), so each wave streams distinct
//     data and needs no barrier inside the K loop;
//   * every wave copies its own K-blocks (all 16*MI rows of A, 16*NI rows of
//     B) straight into a private LDS region with bounds-checked buffer->LDS
//     loads and waits for them with its own vmcnt.  B, the bytes that come
//     from HBM, runs two K-blocks ahead (three stages) and is copied with the
//     non-temporal cache policy (read once); A, which every workgroup
//     re-reads from L2, runs one ahead (two stages);
//   * the four per-wave partial sums are added through LDS in a fixed order
//     (wave 0 + 1 + 2 + 3) before the single rounding to BF16 / FP32, so the
//     result is bitwise repeatable.
#pragma once

#include "gemm_f16mma.hpp"

namespace dg {

// One few-rows problem: rows [0, M) of A / sA / C, one expert's B and sB.
struct SkinnyJob {
  const uint8_t* A;       // [M][K]
  const float* sA;        // [1][Kb] (one row block), or [M][Kb] with ROW_SA
  const uint8_t* B;       // [N][K]
  const float* sB;        // [ceil(N/128)][Kb]; Kb = ceil(K/128)
  void* C;                // [M][N]
  int M, N, K;
};

// Row stride (floats) of the partial sums in the final reduction: the tile's
// 16 NI columns plus 4, so that the 16-byte stores of 8 consecutive lanes
// (rows r .. r + 7 of one column piece) hit 8 distinct 16-byte positions of a
// 128-byte window (rows 16 NI * 4 bytes apart would give 2 or 4 for NI = 3
// or 1: 4- and 2-way bank conflicts).
template <int NI>
constexpr int skinny_red_ld() { return 16 * NI + 4; }

// LDS bytes of gemm_skinny_body: per wave A in 2 stages, B in 3, row scales
// in 2; reused for the partial sums of the final reduction.
template <int MI, int NI, bool ROW_SA>
constexpr int skinny_lds_bytes() {
  constexpr int wave = 2 * 16 * MI * KBLK + 3 * 16 * NI * KBLK + (ROW_SA ? 2 * 256 : 0);
  constexpr int red = 4 * 16 * MI * skinny_red_ld<NI>() * 4;
  return 4 * wave > red ? 4 * wave : red;
}

// The 16*NI columns from n0 of a few-rows problem, in the workgroup's LDS
// buffer `lds` (skinny_lds_bytes bytes, 16-byte aligned).  ROW_SA: sA holds
// one scale per row and K-block ([M][Kb]).
// NT_C: C is written with non-temporal stores (the dense few-rows kernel,
// whose workgroups all store at the end of its single round).
template <int MI, int NI, bool OUT_BF16, int FA = FMT_E4M3, int FB = FMT_E4M3, bool ROW_SA = false,
          bool NT_C = false>
__device__ __forceinline__ void gemm_skinny_body(const SkinnyJob& p, const int n0, uint8_t* lds) {
  constexpr int NW = 4;                         // waves, each a quarter of the K-blocks
  constexpr int RM = 16 * MI, CN = 16 * NI;     // rows / columns of the workgroup tile
  constexpr int A_BYTES = RM * KBLK, B_BYTES = CN * KBLK;
  constexpr int S_BYTES = ROW_SA ? 256 : 0;     // 64 row scales of one K-block
  constexpr int WAVE_LDS = 2 * A_BYTES + 3 * B_BYTES + 2 * S_BYTES;   // A: 2 stages, B: 3, sA: 2
  constexpr int A_CH = RM / 8, B_CH = CN / 8;   // 1 KB copy chunks per K-block
  constexpr int A_OPS = A_CH + (ROW_SA ? 1 : 0); // A copy instructions per K-block (+ its row scales)
  static_assert(2 * B_CH + A_OPS < 64, "vmcnt range");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int M = p.M, N = p.N, K = p.K;
  const int Kb = (K + KBLK - 1) / KBLK;         // the last K-block may be partial
  const int Nb = (N + KBLK - 1) / KBLK;

  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* sAr = (cfloat*)(p.sA);                // M <= 64: one row block
  int nbk[NI];
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) nbk[ni] = min((n0 + 16 * ni) / KBLK, Nb - 1);

  const i32x4 rA = make_rsrc(p.A, uint32_t(M) * uint32_t(K));
  const i32x4 rB = make_rsrc(p.B + (size_t)n0 * K, uint32_t(min(N - n0, CN)) * uint32_t(K));
  // chunk c: LDS rows 8c .. 8c+7; lane L fills row 8c + L/8 slot L%8 with
  // granule (L%8) ^ f(row), f(row) = (L/8) ^ (c & 1)  (see swz16)
  const int lr = lane >> 3;
  const int g_even = ((lane & 7) ^ lr) * 16, g_odd = ((lane & 7) ^ lr ^ 1) * 16;   // source columns
  const uint32_t lane_even = uint32_t(lr * K + g_even);
  const uint32_t lane_odd = uint32_t(lr * K + g_odd);
  // offsets of K-block kb; a granule past K (partial last block) reads as zeros
  auto off_even = [&](int kb) {
    return opaque(kb * KBLK + g_even < K ? lane_even + uint32_t(kb * KBLK) : kOutOfRange);
  };
  auto off_odd = [&](int kb) {
    return opaque(kb * KBLK + g_odd < K ? lane_odd + uint32_t(kb * KBLK) : kOutOfRange);
  };
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
      uint32_t(reinterpret_cast<uintptr_t>(static_cast<void*>(lds))) + uint32_t(wave * WAVE_LDS));

  // row scales (ROW_SA): lane L copies sA[L][kb] (rows past M read as zeros)
  i32x4 rS{};
  if constexpr (ROW_SA) rS = make_rsrc(p.sA, uint32_t(M) * uint32_t(Kb) * 4u);
  const uint32_t s_lane = uint32_t(lane * Kb * 4);
  constexpr int S_OFF = 2 * A_BYTES + 3 * B_BYTES;   // wave LDS offset of the scale stages

  // wave LDS: [A stage 0][A stage 1][B stage 0][B stage 1][B stage 2] ([sA stage 0][sA stage 1])
  auto issue_a = [&](int kb, int stage) {
    const uint32_t ev = off_even(kb);
    const uint32_t od = off_odd(kb);
    const uint32_t base = lds_wave + uint32_t(stage * A_BYTES);
#pragma unroll
    for (int c = 0; c < A_CH; ++c)
      copy16_to_lds(rA, ((c & 1) ? od : ev) + uint32_t(8 * c * K), base + uint32_t(c * 1024));
    if constexpr (ROW_SA)
      copy4_to_lds(rS, s_lane + uint32_t(kb * 4), lds_wave + uint32_t(S_OFF + stage * S_BYTES));
  };
  auto issue_b = [&](int kb, int stage) {
    const uint32_t ev = off_even(kb);
    const uint32_t od = off_odd(kb);
    const uint32_t base = lds_wave + uint32_t(2 * A_BYTES + stage * B_BYTES);
#pragma unroll
    for (int c = 0; c < B_CH; ++c)
      copy16_to_lds_nt(rB, ((c & 1) ? od : ev) + uint32_t(8 * c * K), base + uint32_t(c * 1024));
  };

  v4f acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int q = lane >> 4, r16 = lane & 15;
  const int off0 = r16 * KBLK + swz16(r16, 2 * q) * 16;
  const int off1 = r16 * KBLK + swz16(r16, 2 * q + 1) * 16;
  const uint8_t* lw = lds + wave * WAVE_LDS;

  // Issue order per iteration j (K-block kb_j = wave + 4j): A(kb_{j+1}) then
  // B(kb_{j+2}).  A(kb_j) and B(kb_j) are complete once at most
  // B(kb_{j+1}) + A(kb_{j+1}) + B(kb_{j+2}) copies are still outstanding.
  int j = 0, bstage = 0;
  if (wave < Kb && !kSingleStage) {
    issue_a(wave, 0);
    issue_b(wave, 0);
    if (wave + NW < Kb) issue_b(wave + NW, 1);
  }
  for (int kb = wave; kb < Kb; kb += NW, ++j) {
    const int astage = kSingleStage ? 0 : j & 1;
    const float sa = ROW_SA ? 1.f : float(sAr[kb]);
    float sb[NI];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) sb[ni] = ((cfloat*)p.sB)[(size_t)nbk[ni] * Kb + kb];
    if constexpr (kSingleStage) {
      // this K-block into stage 0, once the previous one's LDS reads have
      // returned (s_waitcnt lgkmcnt(0))
      __builtin_amdgcn_s_waitcnt(0xC07F);
      issue_a(kb, 0);
      issue_b(kb, 0);
      wait_vmem_n<0>();
    } else if (kb + 2 * NW < Kb) {
      issue_a(kb + NW, astage ^ 1);
      issue_b(kb + 2 * NW, bstage == 0 ? 2 : bstage - 1);
      wait_vmem_n<2 * B_CH + A_OPS>();
    } else {
      if (kb + NW < Kb) issue_a(kb + NW, astage ^ 1);
      wait_vmem_n<0>();
    }
    const uint8_t* la = lw + astage * A_BYTES;
    const uint8_t* lb = lw + 2 * A_BYTES + bstage * B_BYTES;
    float sa_m[MI];                               // A scale of row group mi
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) sa_m[mi] = sa;
    if constexpr (ROW_SA) {
      const float* ls = reinterpret_cast<const float*>(lw + S_OFF + astage * S_BYTES);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) sa_m[mi] = ls[16 * mi + r16];
    }
    bstage = kSingleStage ? 0 : bstage == 2 ? 0 : bstage + 1;
    v8h af[MI][4];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int4 x0 = *reinterpret_cast<const int4*>(la + off0 + mi * 16 * KBLK);
      const int4 x1 = *reinterpret_cast<const int4*>(la + off1 + mi * 16 * KBLK);
      fp8x32_to_f16<FA>(x0, x1, af[mi]);
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int4 y0 = *reinterpret_cast<const int4*>(lb + off0 + ni * 16 * KBLK);
      const int4 y1 = *reinterpret_cast<const int4*>(lb + off1 + ni * 16 * KBLK);
      v8h bf[4];
      fp8x32_to_f16<FB>(y0, y1, bf);
      v4f part[MI];
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          part[mi] = mfma16_f16(bf[st], af[mi][st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : part[mi]);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const float s = sa_m[mi] * sb[ni];      // fp32(sA * sB) of this row group and K-block
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][ni][r] = __builtin_fmaf(s, part[mi][r], acc[mi][ni][r]);
      }
    }
  }

  // ---- fixed-order reduction of the four partial sums ----------------------
  __syncthreads();                              // every wave is done with its stages
  constexpr int LD = skinny_red_ld<NI>();
  float* red = reinterpret_cast<float*>(lds);   // [wave][RM][LD]
#pragma unroll
  for (int mi = 0; mi < MI; ++mi)
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      // lane holds rows mi*16 + r16, columns ni*16 + 4q + 0..3
      float* dst = red + (wave * RM + mi * 16 + r16) * LD + ni * 16 + 4 * q;
      *reinterpret_cast<float4*>(dst) = float4{acc[mi][ni][0], acc[mi][ni][1], acc[mi][ni][2], acc[mi][ni][3]};
    }
  __syncthreads();
  constexpr int CH8 = CN / 8;                   // 8-column chunks per row
  for (int c = threadIdx.x; c < RM * CH8; c += 64 * NW) {
    const int m = c / CH8, n8 = (c % CH8) * 8;
    const int n = n0 + n8;
    if (m >= M || n >= N) continue;
    float v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float* src = red + (w * RM + m) * LD + n8;
      const float4 a = *reinterpret_cast<const float4*>(src);
      const float4 b = *reinterpret_cast<const float4*>(src + 4);
      v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
      v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
    }
    store_row_span<OUT_BF16, 8, NT_C>(p.C, size_t(m) * N, n, N, v);
  }
}

template <int MI, int NI, bool OUT_BF16, int FA, int FB, bool ROW_SA>
__device__ __forceinline__ void gemm_skinny_dense(const GemmArgs& p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[skinny_lds_bytes<MI, NI, ROW_SA>()];
  const SkinnyJob j{p.A, p.sA, p.B, p.sB, p.C, p.M, p.N, p.K};
  gemm_skinny_body<MI, NI, OUT_BF16, FA, FB, ROW_SA, true>(j, int(blockIdx.x) * 16 * NI, lds);
}

// Grouped GEMM over unpadded expert segments (rows [o_e, o_{e+1}) of A and C
// belong to expert e, any o_e), one A scale per row.  Workgroup b takes
// expert e = b / n_tiles and column slab b % n_tiles.  The chunk height is
// chosen per expert from its row count (16, 32 or 64 rows, a uniform branch),
// so an expert with at most 64 rows streams its slab of B_e exactly once;
// longer segments are walked in chunks of 64 rows, each streaming the slab
// again.  Experts without rows cost two offset reads.  Offsets are clamped to
// [0, M] so that inconsistent offsets cannot address outside A or C.
template <int NI, bool OUT_BF16, int FA, int FB>
__device__ __forceinline__ void gemm_skinny_segments(const GemmArgs& p) {
  constexpr int L1 = skinny_lds_bytes<1, NI, true>(), L2 = skinny_lds_bytes<2, NI, true>();
  constexpr int L4 = skinny_lds_bytes<4, NI, true>();
  constexpr int L12 = L1 > L2 ? L1 : L2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[L12 > L4 ? L12 : L4];
  const int e = int(blockIdx.x) / p.n_tiles;
  const int n0 = (int(blockIdx.x) - e * p.n_tiles) * 16 * NI;
  typedef const __attribute__((address_space(4))) int32_t cint;
  const int lo = min(max(int(((cint*)p.offs)[e]), 0), p.M);
  const int hi = min(max(int(((cint*)p.offs)[e + 1]), lo), p.M);
  const int N = p.N, K = p.K, Kb = (K + KBLK - 1) / KBLK, Nb = (N + KBLK - 1) / KBLK;
  const size_t c_row = size_t(N) * (OUT_BF16 ? 2 : 4);
  auto job = [&](int r0, int rows) {
    return SkinnyJob{p.A + size_t(r0) * K, p.sA + size_t(r0) * Kb, p.B + size_t(e) * N * K,
                     p.sB + size_t(e) * Nb * Kb, static_cast<uint8_t*>(p.C) + size_t(r0) * c_row, rows, N, K};
  };
  const int len = hi - lo;
  if (len <= 0) return;
  if (len <= 16) {
    gemm_skinny_body<1, NI, OUT_BF16, FA, FB, true>(job(lo, len), n0, lds);
  } else if (len <= 32) {
    gemm_skinny_body<2, NI, OUT_BF16, FA, FB, true>(job(lo, len), n0, lds);
  } else {
    for (int r0 = lo; r0 < hi; r0 += 64) {
      if (r0 != lo) __syncthreads();           // LDS of the previous chunk's reduction is free
      gemm_skinny_body<4, NI, OUT_BF16, FA, FB, true>(job(r0, min(hi - r0, 64)), n0, lds);
    }
  }
}

#define DG_SKINNY_KERNEL_DEF(NAME, MI, NI, BF16, FA, FB, RS) \
  __global__ __launch_bounds__(256, 1) void NAME(GemmArgs p) { gemm_skinny_dense<MI, NI, BF16, FA, FB, RS>(p); }
#define DG_SKINNY_KERNEL_DECL(NAME, MI, NI, BF16, FA, FB, RS) \
  __global__ __launch_bounds__(256, 1) void NAME(GemmArgs p);
#define DG_SKINNY_SHAPE(K, ROWS, COLS, MI, NI, SFX, FA, FB, RS)               \
  K(dg_skinny_m##ROWS##_n##COLS##_bf16##SFX, MI, NI, true, FA, FB, RS)        \
  K(dg_skinny_m##ROWS##_n##COLS##_f32##SFX, MI, NI, false, FA, FB, RS)
#define DG_SKINNY_ROWS(K, SFX, FA, FB, RS)                                                          \
  DG_SKINNY_SHAPE(K, 64, 48, 4, 3, SFX, FA, FB, RS) DG_SKINNY_SHAPE(K, 64, 16, 4, 1, SFX, FA, FB, RS) \
  DG_SKINNY_SHAPE(K, 32, 48, 2, 3, SFX, FA, FB, RS) DG_SKINNY_SHAPE(K, 32, 16, 2, 1, SFX, FA, FB, RS) \
  DG_SKINNY_SHAPE(K, 16, 48, 1, 3, SFX, FA, FB, RS) DG_SKINNY_SHAPE(K, 16, 16, 1, 1, SFX, FA, FB, RS)
#define DG_SEG_KERNEL_DEF(NAME, NI, BF16, FA, FB) \
  __global__ __launch_bounds__(256, 1) void NAME(GemmArgs p) { gemm_skinny_segments<NI, BF16, FA, FB>(p); }
#define DG_SEG_KERNEL_DECL(NAME, NI, BF16, FA, FB) __global__ __launch_bounds__(256, 1) void NAME(GemmArgs p);
#define DG_SEG_SHAPE(K, COLS, NI, SFX, FA, FB)                \
  K(dg_segments_n##COLS##_bf16##SFX, NI, true, FA, FB)        \
  K(dg_segments_n##COLS##_f32##SFX, NI, false, FA, FB)
#define DG_FEW_ROWS_FORMATS(GROUP, SFX, FA, FB)                                \
  DG_SKINNY_ROWS(DG_KERNEL(DG_SKINNY_KERNEL, GROUP), SFX, FA, FB, false)      \
  DG_SKINNY_ROWS(DG_KERNEL(DG_SKINNY_KERNEL, GROUP), SFX##_rs, FA, FB, true)  \
  DG_SEG_SHAPE(DG_KERNEL(DG_SEG_KERNEL, GROUP), 48, 3, SFX, FA, FB)           \
  DG_SEG_SHAPE(DG_KERNEL(DG_SEG_KERNEL, GROUP), 16, 1, SFX, FA, FB)
DG_FEW_ROWS_FORMATS(FMT_44, , FMT_E4M3, FMT_E4M3)
DG_FEW_ROWS_FORMATS(FMT_55, _a5b5, FMT_E5M2, FMT_E5M2)
DG_FEW_ROWS_FORMATS(FMT_45, _a4b5, FMT_E4M3, FMT_E5M2)
DG_FEW_ROWS_FORMATS(FMT_54, _a5b4, FMT_E5M2, FMT_E4M3)
#undef DG_FEW_ROWS_FORMATS
#undef DG_SEG_SHAPE
#undef DG_SEG_KERNEL_DECL
#undef DG_SEG_KERNEL_DEF
#undef DG_SKINNY_ROWS
#undef DG_SKINNY_SHAPE
#undef DG_SKINNY_KERNEL_DECL
#undef DG_SKINNY_KERNEL_DEF

}  // namespace dg
