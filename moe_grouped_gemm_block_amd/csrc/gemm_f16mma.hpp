// FP8 block-scaled GEMM kernel for gfx950 (dense and MoE-grouped).
//
// What it computes: for every 128-wide K-block, the exact products of the
// E4M3 operands summed with FP32-grade accumulation, rescaled in FP32 by
// fp32(sA * sB) of that block and added to an FP32 accumulator (block-wise
// scaling of the DeepGEMM FP8-for-MoE page, 2kiu.com/news/5461879, sections
// 2.1 and 3.3).
//
// Why FP16 matrix cores.  On gfx950 the FP8 MFMA sums the products of every
// group of 8 consecutive K elements inside a window of about 14 bits below
// the largest product of the group and drops whatever lies below it; on
// Gaussian blocks that alone reaches ~1.7e-5 of sum|a b|, and far more on
// blocks with a wide spread of magnitudes.  The FP16 MFMA keeps a 24-bit
// window, i.e. it accumulates like FP32.  Every E4M3 value is exactly an
// FP16 value, so converting the fragments (v_cvt_scalef32_pk_f16_fp8, two
// values per instruction, scale 1) loses nothing and the FP16 matrix cores
// then deliver the block partials that the definition asks for.  (The pages'
// Hopper kernels promote FP8 tensor-core partials to FP32 registers every
// K-block for the same kind of reason: FP8 MMA accumulation is narrow.)
//
// Structure (tiling of the DeepGEMM FP8 kernel write-up, demingchina.com/
// news/60142, sections 2.3 and 3.3-4.3, re-planned for CDNA4):
//   * a workgroup of NWM x NWN waves computes a (64 NWM) x (WN NWN) tile of
//     C; every wave owns a 64 x WN sub-tile (16 x 16 MFMA tiles 4 x WN/16),
//     WN = 128, or 64 for the narrow tiles that small grids use.  With 8
//     waves, two share each SIMD so that one wave's vector work (format
//     conversion, rescale) overlaps the other's matrix-core work;
//   * A and B stay FP8 in HBM and LDS.  Each K-block's tiles are copied
//     straight into LDS by bounds-checked buffer loads (16 bytes per lane, no
//     VGPR staging; rows past the matrix edge read as zeros), two stages:
//     the next K-block streams in while the current one is multiplied;
//   * inside a 128-byte LDS row the 16-byte granules are XOR-swizzled with a
//     pattern that repeats every 16 rows (see swz16), so fragment reads are
//     spread over the banks and every read of a wave is one base register
//     plus an immediate offset;
//   * B rows are permuted on their way into LDS so that, with B as the MFMA's
//     first operand, each lane ends up holding four runs of 8 consecutive
//     columns of one output row, 32 columns apart, and the four lanes of a
//     row hold adjacent runs: every 16-byte store instruction of the
//     epilogue writes whole 64-byte pieces of C rows (with 16-byte pieces
//     64 bytes apart, writing the C of a 4096 x 4096 BF16 problem took
//     ~12 us instead of ~7 us);
//   * per K-block and wave: FP8 fragments -> FP16 in registers, 4 chained
//     16x16x32 FP16 MFMAs per 16 x 16 output tile give the block partial P,
//     then acc = fma(sA*sB, P, acc) in FP32.  Wave sub-tiles never straddle
//     a 128 x 128 scale block, so sA*sB is one scalar per wave and K-block
//     (with per-row A scales, one factor per row group: see ROW_SA);
//   * the last K-block may be partial (K a multiple of 16): its copies past
//     K read as zeros;
//   * tiles are ordered so that each XCD (own L2) works on a compact group of
//     row and column tiles.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace dg {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// Operand code formats.
constexpr int FMT_E4M3 = 0;   // OCP E4M3FN
constexpr int FMT_E5M2 = 1;   // E5M2

// Four FP8 bytes -> four FP16 values (exact), as two packed pairs.  E4M3:
// the hardware conversion (scale 1).  E5M2: an E5M2 byte is the high byte
// of the IEEE half of the same value (same sign, 5-bit exponent with bias
// 15, the first 2 mantissa bits; subnormals, infinities and NaN included),
// so the conversion only moves bytes.
template <int FMT = FMT_E4M3>
__device__ __forceinline__ void fp8x4_to_f16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  if constexpr (FMT == FMT_E4M3) {
    const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w), 1.0f, false);
    const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(static_cast<int>(w), 1.0f, true);
    lo = __builtin_bit_cast(uint32_t, a);
    hi = __builtin_bit_cast(uint32_t, b);
  } else {
    // v_perm_b32 byte selectors (byte 3 .. byte 0 of the result): 0..3 pick
    // a byte of w, 0x0C gives 0x00
    lo = __builtin_amdgcn_perm(0u, w, 0x010C000Cu);   // [w.b1, 0, w.b0, 0]
    hi = __builtin_amdgcn_perm(0u, w, 0x030C020Cu);   // [w.b3, 0, w.b2, 0]
  }
}

// 32 FP8 bytes of one fragment row -> the four FP16 MFMA operands of the
// K-block (operand s holds bytes 8s .. 8s+7).
template <int FMT = FMT_E4M3>
__device__ __forceinline__ void fp8x32_to_f16(const int4& r0, const int4& r1, v8h out[4]) {
  const uint32_t w[8] = {uint32_t(r0.x), uint32_t(r0.y), uint32_t(r0.z), uint32_t(r0.w),
                         uint32_t(r1.x), uint32_t(r1.y), uint32_t(r1.z), uint32_t(r1.w)};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint32_t h[4];
    fp8x4_to_f16<FMT>(w[2 * s], h[0], h[1]);
    fp8x4_to_f16<FMT>(w[2 * s + 1], h[2], h[3]);
    out[s] = __builtin_bit_cast(v8h, (uint4{h[0], h[1], h[2], h[3]}));
  }
}

// MFMA operand st (bytes 8st .. 8st+7 of a lane's 32) of the raw fragment
// pair r0 (bytes 0..15), r1 (bytes 16..31), as eight FP16 values.
template <int FMT = FMT_E4M3>
__device__ __forceinline__ v8h fp8_operand(const int4& r0, const int4& r1, int st) {
  const int4& r = st < 2 ? r0 : r1;
  const uint32_t w0 = uint32_t((st & 1) ? r.z : r.x), w1 = uint32_t((st & 1) ? r.w : r.y);
  uint32_t h[4];
  fp8x4_to_f16<FMT>(w0, h[0], h[1]);
  fp8x4_to_f16<FMT>(w1, h[2], h[3]);
  return __builtin_bit_cast(v8h, (uint4{h[0], h[1], h[2], h[3]}));
}

__device__ __forceinline__ v4f mfma16_f16(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Returns x unchanged through an empty (non-volatile) asm, which the
// optimiser cannot see through: used on per-K-block copy offsets so that they
// are not strength-reduced into one long-lived register per copy chunk.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm("" : "+v"(x));
  return x;
}

// Lane index recomputed on the spot (keeps it from living across the K loop).
__device__ __forceinline__ int lane_id() {
  return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
}

// s_waitcnt vmcnt(0) (expcnt / lgkmcnt left at their maxima): waits for this
// wave's outstanding global->LDS copies.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt at their maxima (n < 64).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | 0x0F70);
}

// Swizzle of the 16-byte granule g of LDS row r: slot g ^ f(r) with
// f(r) = (r & 7) ^ ((r >> 3) & 1).  Within any 16 consecutive rows starting
// at a multiple of 16, (r & 1, f(r)) takes 16 distinct values, so the 16
// lanes that read one granule of 16 rows hit 16 distinct 16-byte bank groups
// of a 256-byte window (and 8 distinct ones per 8 rows); f depends on r mod
// 16 only.  This is the 8-row XOR swizzle of the DeepGEMM FP8 kernel
// write-up (section 4.2) re-derived for 16-byte granules and 64-lane reads.
__device__ __forceinline__ int swz16(int r, int g) { return g ^ ((r & 7) ^ ((r >> 3) & 1)); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resource (stride 0) over `bytes` bytes at `base`: loads at
// offsets >= bytes return zeros instead of touching memory.
// Every field goes through readfirstlane: the descriptor must sit in SGPRs.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane(int(uint32_t(a)));
  r[1] = __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffffu));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(int(bytes));                          // num_records
  r[3] = 0x00020000;                                                          // 32-bit data format
  return r;
}

// 16 bytes per lane from buffer `rsrc` at byte offset `voff` straight into
// LDS at `lds_base` + 16 * lane (lds_base is wave-uniform, passed in M0).
// Written as inline assembly on purpose: the compiler then does not treat
// the copy as an LDS store that every later LDS read must wait for -- the
// copies always target the stage that is not being read, and the kernel
// waits for them itself (s_waitcnt vmcnt(0) + barrier) before switching.
__device__ __forceinline__ void copy16_to_lds(const i32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
               : "memory");
}

// The same copy with the non-temporal cache policy, for data read exactly
// once (the few-rows kernel's B stream): 4.8 % faster on M = 64, N = 12288,
// K = 4096, where B is 48 MB that no other workgroup reads again.
__device__ __forceinline__ void copy16_to_lds_nt(const i32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
               : "memory");
}

// 4 bytes per lane from buffer `rsrc` at byte offset `voff` into LDS at
// `lds_base` + 4 * lane (same conventions as copy16_to_lds).
__device__ __forceinline__ void copy4_to_lds(const i32x4& rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc), "{m0}"(lds_base)
               : "memory");
}

struct GemmArgs {
  const uint8_t* A;       // [M][K]
  const float* sA;        // [ceil(M/128)][Kb], or [M][Kb] with per-row scales
  const uint8_t* B;       // [G][N][K]
  const float* sB;        // [G][ceil(N/128)][Kb]; Kb = ceil(K/128)
  void* C;                // [M][N]
  const int32_t* offs;    // [G+1] device, or nullptr for dense
  // grouped, optional: [G] real rows per expert; rows [offs[e] + counts[e],
  // offs[e+1]) are padding, written as zeros without their A rows being used
  const int32_t* counts;
  int G;
  int M, N, K;
  int m_tiles, n_tiles;    // tiles of this launch
  int m_tile0;            // first row tile of this launch, in tiles of the kernel's height (a launch may cover a row range)
  // Split K (tiled kernels only): with splits > 1 the grid holds `splits`
  // copies of the tile grid; copy s sums K-blocks [s Kb / splits,
  // (s + 1) Kb / splits) of every tile and stores its FP32 partial into
  // ws[s][row - m_tile0 * tile height][column] (row stride ws_ld, a
  // multiple of 4 that is at least N; ws_rows rows per copy) instead of C.
  // splitk_reduce then adds the copies in order s = 0, 1, ... into C.
  int splits;
  float* ws;
  int ws_ld, ws_rows;
};

// First padding row of the segment of expert e (grouped, with per-expert
// real row counts), else M: rows [offs[e] + counts[e], offs[e+1]) are
// padding.  Wave-uniform.
__device__ __forceinline__ int padding_start(const GemmArgs& p, int e) {
  if (p.offs == nullptr || p.counts == nullptr) return p.M;
  const int seg0 = p.offs[e], len = p.offs[e + 1] - seg0;
  return __builtin_amdgcn_readfirstlane(seg0 + min(max(p.counts[e], 0), max(len, 0)));
}

// K-blocks [kb_begin, kb_end) of split s out of S (every split gets
// floor or ceil of Kb / S; a split may be empty when S > Kb).
__device__ __forceinline__ int split_kb(int s, int S, int Kb) { return int((int64_t(s) * Kb) / S); }

// Tile order: blockIdx -> (m-tile, n-tile).  Workgroups are dealt to the 8
// XCDs round-robin (block b runs on XCD b % 8), so block b is given tile t
// from a contiguous range per XCD: XCD x owns tiles [start_x, start_x +
// count_x), the first T % 8 XCDs one tile more than the others.  Inside the
// range, tiles walk a group of GROUP_M row tiles column by column, so the
// tiles that run together on one XCD share A rows and B columns in its L2
// (and, for grouped problems, the same experts' weights).
template <int GROUP_M>
__device__ __forceinline__ void tile_of(int bid, int m_tiles, int n_tiles, int& tm, int& tn) {
  const int T = m_tiles * n_tiles;
  const int xcd = bid & 7, local = bid >> 3;
  const int base = T >> 3, extra = T & 7;
  const int t = xcd < extra ? xcd * (base + 1) + local : extra * (base + 1) + (xcd - extra) * base + local;
  const int per_group = GROUP_M * n_tiles;
  const int g = t / per_group;
  const int first_m = g * GROUP_M;
  const int gsize = min(GROUP_M, m_tiles - first_m);
  const int r = t - g * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// ROW_SA: sA holds one scale per row and K-block ([rows][Kb], the 1 x 128
// per-token granularity) instead of one per 128 x 128 block.  Each lane then
// loads the scales of its four rows one K-block ahead with ordinary vector
// loads: the loop drains every copy (vmcnt(0)) at the end of each K-block
// anyway, so waiting for these loads costs nothing, and no LDS is needed.
template <int NWM, int NWN, bool OUT_BF16, int FA = FMT_E4M3, int FB = FMT_E4M3, bool ROW_SA = false,
          int WN = 128>
__device__ __forceinline__ void gemm_f16mma_body(const GemmArgs& p) {
  static_assert(WN == 128 || WN == 64, "wave sub-tile width");
  constexpr int WM = 64;                       // wave sub-tile: WM x WN
  constexpr int MI = WM / 16, NI = WN / 16;    // 16x16 MFMA tiles per wave
  constexpr int NW = NWM * NWN;                // waves per workgroup
  constexpr int BM = NWM * WM, BN = NWN * WN;  // workgroup tile
  constexpr int A_BYTES = BM * KBLK, B_BYTES = BN * KBLK;
  constexpr int A_CH = BM / 8 / NW, B_CH = BN / 8 / NW;   // 1 KB copy chunks per wave
  static_assert(A_CH * 8 * NW == BM && B_CH * 8 * NW == BN, "chunking");
  static_assert(NW % 2 == 0, "chunk parity per wave assumes an even wave count");
  // LDS: [A stage 0][A stage 1][B stage 0][B stage 1]
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (A_BYTES + B_BYTES)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // split of K this workgroup sums (0 without a split) and its tile
  const int T = p.m_tiles * p.n_tiles;
  const int split = p.splits > 1 ? int(blockIdx.x) / T : 0;
  int tm, tn;
  tile_of<8>(int(blockIdx.x) - split * T, p.m_tiles, p.n_tiles, tm, tn);
  const int m0 = (p.m_tile0 + tm) * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int Kb = (K + KBLK - 1) / KBLK;          // the last K-block may be partial
  const int Nb = (N + KBLK - 1) / KBLK;
  const int S = max(p.splits, 1);
  const int kb0 = split_kb(split, S, Kb);

  int e = 0;
  if (p.offs != nullptr) {
    e = find_group(p.offs, p.G, m0);
    if (e >= p.G) return;                      // uniform across the workgroup
  }
  // rows from real_end on are padding; a tile of padding rows only runs no
  // K-blocks (its epilogue writes zeros)
  const int real_end = padding_start(p, e);
  const int kb1 = m0 < real_end ? split_kb(split + 1, S, Kb) : kb0;
  const int wm = (wave / NWN) * WM;            // wave sub-tile origin in the tile
  const int wn = (wave % NWN) * WN;
  // scale rows of this wave (clamped: a wave wholly past the edge stores nothing)
  const int mb = min((m0 + wm) / KBLK, (M - 1) / KBLK);
  const int nb = min((n0 + wn) / KBLK, Nb - 1);
  // Scales are read through the constant address space so that they become
  // scalar loads (counted apart from the vector-memory copies into LDS).
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* sAr = (cfloat*)(p.sA + (ROW_SA ? 0 : (size_t)mb * Kb));   // (unused with ROW_SA)
  cfloat* sBr = (cfloat*)(p.sB + ((size_t)e * Nb + nb) * Kb);

  // ---- global -> LDS copies --------------------------------------------------
  // Buffer resources start at the tile's first row and end at the matrix
  // edge, so rows past M (or N) come back as zeros.
  const i32x4 rA = make_rsrc(p.A + (size_t)m0 * K, uint32_t(min(M - m0, BM)) * uint32_t(K));
  const i32x4 rB = make_rsrc(p.B + ((size_t)e * N + n0) * K, uint32_t(min(N - n0, BN)) * uint32_t(K));
  // Chunk c = 1 KB = LDS rows 8c .. 8c+7 of a tile; lane L fills row 8c + L/8,
  // slot L%8, with granule (L%8) ^ f(row).  This wave copies chunks
  // c = wave + NW i; all of them have the parity of `wave`, so f(row) =
  // (L/8) ^ (wave & 1) and one per-lane offset serves every chunk.
  const int lr = lane >> 3;
  const int gsl = ((lane & 7) ^ lr ^ (wave & 1)) * 16;
  const uint32_t a_lane = uint32_t(lr * K + gsl);
  // B: LDS row r = 8c + L/8 holds, inside column half h = r / 128, operand
  // row ii = r % 16 of MFMA column tile ni = (r % 128) / 16, i.e. the tile
  // row 128 h + 32 (ni / 2) + 8 (ii / 4) + 4 (ni % 2) + ii % 4.  With
  // ii = 8 (c % 2) + L/8, the lane contributes 8 (L / 32) + (L/8) % 4.
  // With 64-column waves the two waves of a 128-column group hold tiles
  // ni = 0..3 and 4..7 of this numbering, each its own 64 columns.
  const uint32_t b_lane = uint32_t((8 * (lane >> 5) + (lr & 3)) * K + gsl);

  // LDS byte address of the buffer (wave-uniform)
  const uint32_t lds_addr = __builtin_amdgcn_readfirstlane(
      uint32_t(reinterpret_cast<uintptr_t>(static_cast<void*>(lds))));
  auto issue_copies = [&](int kb, int stage) {
    // a granule past K (partial last K-block) reads as zeros: its offset is
    // pushed past the buffer end (all offsets stay below 2^32)
    const bool k_in = kb * KBLK + gsl < K;
    const uint32_t a_kb = opaque(k_in ? a_lane + uint32_t(kb * KBLK) : kOutOfRange);
    const uint32_t b_kb = opaque(k_in ? b_lane + uint32_t(kb * KBLK) : kOutOfRange);
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
      const int c = wave + NW * i;
      const uint32_t voff = a_kb + uint32_t(8 * c * K);
      copy16_to_lds(rA, voff, lds_addr + uint32_t(stage * A_BYTES + c * 1024));
    }
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      const int c = wave + NW * i;
      const int row = 128 * (c >> 4) + 32 * ((c & 15) >> 2) + 16 * (c & 1) + 4 * ((c >> 1) & 1);
      const uint32_t voff = b_kb + uint32_t(row * K);
      copy16_to_lds(rB, voff, lds_addr + uint32_t(2 * A_BYTES + stage * B_BYTES + c * 1024));
    }
  };

  v4f acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int q = lane >> 4;                     // 32-byte K chunk of this lane
  const int r16 = lane & 15;
  // fragment read offsets (bytes) of this lane inside a tile's wave rows
  const int a_off0 = (wm + r16) * KBLK + swz16(r16, 2 * q) * 16;
  const int a_off1 = (wm + r16) * KBLK + swz16(r16, 2 * q + 1) * 16;
  const int b_off0 = (wn + r16) * KBLK + swz16(r16, 2 * q) * 16;
  const int b_off1 = (wn + r16) * KBLK + swz16(r16, 2 * q + 1) * 16;

  if (kb1 > kb0) {
    issue_copies(kb0, 0);
    wait_vmem();
    __syncthreads();
  }

  // ROW_SA: lane L loads the scale of row wm + L (the wave's 64 rows, one
  // register), through a buffer that ends at the matrix edge (rows past M
  // read as 0; their output is never stored); each lane then fetches the
  // scales of its rows wm + 16 mi + r16 from lanes 16 mi + r16
  const __amdgpu_buffer_rsrc_t rS = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(p.sA) + (size_t)m0 * Kb, 0,
      ROW_SA ? int(uint32_t(min(M - m0, BM)) * uint32_t(Kb) * 4u) : 0, 0x00020000);
  const uint32_t s_off = uint32_t((wm + lane) * Kb * 4);
  float sa_lane = 0.f;                         // scale of row wm + lane, next K-block
  auto load_row_scales = [&](int kb) {
    sa_lane = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rS, int(s_off + uint32_t(kb * 4)), 0, 0));
  };
  if constexpr (ROW_SA) {
    if (kb1 > kb0) load_row_scales(kb0);
  }

  if (m0 + wm >= real_end) {
    // A wave whose 64 rows are all padding still issues its share of every
    // K-block's copies (they are shared by the workgroup) and passes the
    // same waits and barriers as the others, but computes nothing: its
    // SIMD's other wave then has the matrix core to itself.  (A separate
    // loop: a branch inside the hot loop, or one loop body instantiated
    // twice through a lambda, cost registers there.)
    for (int kb = kb0; kb < kb1; ++kb) {
      const int stage = kSingleStage ? 0 : (kb - kb0) & 1;
      if (kb + 1 < kb1 && !kSingleStage) issue_copies(kb + 1, stage ^ 1);
      if constexpr (kSingleStage) {
        __syncthreads();
        if (kb + 1 < kb1) issue_copies(kb + 1, 0);
      }
      wait_vmem();
      __syncthreads();
    }
  } else {
    float sa_next = kb1 > kb0 && !ROW_SA ? float(sAr[kb0]) : 1.f, sb_next = kb1 > kb0 ? sBr[kb0] : 0.f;
    for (int kb = kb0; kb < kb1; ++kb) {
      const int stage = kSingleStage ? 0 : (kb - kb0) & 1;
      const float s = sa_next * sb_next;         // this K-block's fp32(sA * sB)
      float s_m[MI];                              // the factor of row group mi
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) s_m[mi] = s;
      if constexpr (ROW_SA) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          s_m[mi] = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(4 * (16 * mi + r16),
                                                                           __builtin_bit_cast(int, sa_lane))) *
                    sb_next;
          // consumed before the next copies are issued, so that the wait for
          // these loads cannot fall after (and drain) those copies
          asm volatile("" : "+v"(s_m[mi]));
        }
      }
      if (kb + 1 < kb1) {
        if constexpr (ROW_SA) load_row_scales(kb + 1);   // prefetched one K-block ahead
        else sa_next = sAr[kb + 1];
        sb_next = sBr[kb + 1];
        if constexpr (!kSingleStage) issue_copies(kb + 1, stage ^ 1);
      }
      const uint8_t* la = lds + stage * A_BYTES;
      const uint8_t* lb = lds + 2 * A_BYTES + stage * B_BYTES;

      v8h af[MI][4];
      v8h bf[4];
      v4f part[MI];
      int4 y0, y1;   // raw bytes of the B column tile after the next one
      if constexpr (!ROW_SA) {
        // Raw FP8 fragments, all read before the first wait: A rows
        // wm + 16 mi + r16 (the MFMA's second operand), bytes [32q, 32q+32),
        // and the first two B column tiles.
        int4 xa0[MI], xa1[MI];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          xa0[mi] = *reinterpret_cast<const int4*>(la + a_off0 + mi * 16 * KBLK);
          xa1[mi] = *reinterpret_cast<const int4*>(la + a_off1 + mi * 16 * KBLK);
        }
        y0 = *reinterpret_cast<const int4*>(lb + b_off0);
        y1 = *reinterpret_cast<const int4*>(lb + b_off1);
        int4 z0 = y0, z1 = y1;
        if (NI > 1) {
          z0 = *reinterpret_cast<const int4*>(lb + b_off0 + 16 * KBLK);
          z1 = *reinterpret_cast<const int4*>(lb + b_off1 + 16 * KBLK);
        }
        // Column tile 0, k-step by k-step: each A operand is converted just
        // before its first MFMA, so the matrix core starts after a few
        // conversions instead of after all of A.  The B operands of tile 1 are
        // converted into the registers each k-step frees, and the raw bytes of
        // tile 2 are read into those of tile 0.
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          bf[st] = fp8_operand<FB>(y0, y1, st);
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            af[mi][st] = fp8_operand<FA>(xa0[mi], xa1[mi], st);
            part[mi] = mfma16_f16(bf[st], af[mi][st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : part[mi]);
          }
          if (NI > 1) {
            bf[st] = fp8_operand<FB>(z0, z1, st);
            if (NI > 2 && st == 1) y0 = *reinterpret_cast<const int4*>(lb + b_off0 + 2 * 16 * KBLK);
            if (NI > 2 && st == 3) y1 = *reinterpret_cast<const int4*>(lb + b_off1 + 2 * 16 * KBLK);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * MI + (NI > 1 ? 4 : 2), 0);   // raw reads first
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                     // B operand of tile 0
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);                   // A operand
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                   // 1 MFMA
          }
          if (NI > 1) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);         // B operand of tile 1
        }
      } else {
        // Row-scaled A: one more live register per row group, which leaves no
        // room for the raw fragments of both operands at once (they would be
        // spilled, and reloading a spill inside the loop waits for the copies
        // in flight).  A is converted first, then tile 0 runs as the others do.
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const int4 x0 = *reinterpret_cast<const int4*>(la + a_off0 + mi * 16 * KBLK);
          const int4 x1 = *reinterpret_cast<const int4*>(la + a_off1 + mi * 16 * KBLK);
          fp8x32_to_f16<FA>(x0, x1, af[mi]);
        }
        y0 = *reinterpret_cast<const int4*>(lb + b_off0);
        y1 = *reinterpret_cast<const int4*>(lb + b_off1);
        fp8x32_to_f16<FB>(y0, y1, bf);
        if (NI > 1) {
          y0 = *reinterpret_cast<const int4*>(lb + b_off0 + 16 * KBLK);
          y1 = *reinterpret_cast<const int4*>(lb + b_off1 + 16 * KBLK);
        }
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi)
            part[mi] = mfma16_f16(bf[st], af[mi][st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : part[mi]);
          if (NI > 1) {
            bf[st] = fp8_operand<FB>(y0, y1, st);   // operand st of tile 1
            if (NI > 2 && st == 1) y0 = *reinterpret_cast<const int4*>(lb + b_off0 + 2 * 16 * KBLK);
            if (NI > 2 && st == 3) y1 = *reinterpret_cast<const int4*>(lb + b_off1 + 2 * 16 * KBLK);
          }
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        if (NI > 1) {
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            if (st > 0) {
#pragma unroll
              for (int mi = 0; mi < MI; ++mi) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // 1 VALU (convert)
              }
            } else {
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);     // converts of operand 0
            }
          }
        }
      }
      // Column tiles 1 .. NI-1, software-pipelined: while the MFMAs of tile ni
      // consume operand st, operand st of tile ni+1 is converted into the
      // registers they free, and the FP32 rescale of tile ni-1 is threaded
      // between the first MFMAs of tile ni.  Raw FP8 of tile ni+2 is read from
      // LDS one tile ahead.
#pragma unroll
      for (int ni = 1; ni < NI; ++ni) {
#pragma unroll
        for (int st = 0; st < 4; ++st) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) {
            if (st == 0) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[mi][ni - 1][r] = __builtin_fmaf(s_m[mi], part[mi][r], acc[mi][ni - 1][r]);
            }
            part[mi] = mfma16_f16(bf[st], af[mi][st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : part[mi]);
          }
          if (ni + 1 < NI) {
            bf[st] = fp8_operand<FB>(y0, y1, st);   // operand st of tile ni+1
            if (ni + 2 < NI && st == 1)
              y0 = *reinterpret_cast<const int4*>(lb + b_off0 + (ni + 2) * 16 * KBLK);
            if (ni + 2 < NI && st == 3)
              y1 = *reinterpret_cast<const int4*>(lb + b_off1 + (ni + 2) * 16 * KBLK);
          }
        }
        // pin the interleave: rescale / MFMA alternation, then MFMA / convert
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // 4 VALU (rescale)
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
        }
        if (ni + 1 < NI) {
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            if (st > 0) {
#pragma unroll
              for (int mi = 0; mi < MI; ++mi) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // 1 MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);   // 1 VALU (convert)
              }
            } else {
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);     // converts of operand 0
            }
          }
        }
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mi][NI - 1][r] = __builtin_fmaf(s_m[mi], part[mi][r], acc[mi][NI - 1][r]);
      if constexpr (kSingleStage) {
        __syncthreads();                          // every wave is done with the stage
        if (kb + 1 < kb1) issue_copies(kb + 1, 0);
      }
      wait_vmem();
      __syncthreads();
    }
  }

  // ---- epilogue: column tiles 2j and 2j+1 of a lane hold
  // C[m][n0 + wn + 32 j + 8 q + 0 .. 7]; padding rows get zeros (their first
  // row is looked up again rather than kept in a register through the loop)
  const int pad0 = padding_start(p, p.offs != nullptr ? find_group(p.offs, p.G, m0) : 0);
  const int lane_e = lane_id();
  const int q_e = lane_e >> 4, r16_e = lane_e & 15;
  if (p.splits > 1) {
    // FP32 partial of this split: rows counted from the launch's first row;
    // a vector that starts below N lies inside the padded row (ws_ld >= N
    // rounded up to 4), so whole 16-byte vectors are stored
    float* W = p.ws + (size_t)split * p.ws_rows * p.ws_ld;
    const int r0 = p.m_tile0 * BM;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      const int m = m0 + wm + mi * 16 + r16_e;
      if (m >= M) continue;
      const bool pad = m >= pad0;
      float* row = W + (size_t)(m - r0) * p.ws_ld;
#pragma unroll
      for (int j = 0; j < NI / 2; ++j) {
        const int n = n0 + wn + 32 * j + 8 * q_e;
        const v4f a = pad ? v4f{0.f, 0.f, 0.f, 0.f} : acc[mi][2 * j];
        const v4f b = pad ? v4f{0.f, 0.f, 0.f, 0.f} : acc[mi][2 * j + 1];
        if (n < N) *reinterpret_cast<float4*>(row + n) = float4{a[0], a[1], a[2], a[3]};
        if (n + 4 < N) *reinterpret_cast<float4*>(row + n + 4) = float4{b[0], b[1], b[2], b[3]};
      }
    }
    return;
  }
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = m0 + wm + mi * 16 + r16_e;
    if (m >= M) continue;
    const bool pad = m >= pad0;
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = pad ? 0.f : acc[mi][2 * j][r];
        v[4 + r] = pad ? 0.f : acc[mi][2 * j + 1][r];
      }
      store_row_span<OUT_BF16, 8>(p.C, size_t(m) * N, n0 + wn + 32 * j + 8 * q_e, N, v);
    }
  }
}

// Sum of the split-K partials: C[row0 + r][n] = ((ws[0][r][n] + ws[1][r][n])
// + ...) + ws[S-1][r][n], always in this order (the result does not depend
// on which split finished first), rounded once to the output type.  One
// thread per 8 consecutive columns of a row.
struct ReduceArgs {
  const float* ws;   // [splits][rows][ld]
  void* C;           // [..][N]; rows row0 .. row0 + rows - 1 are written
  int splits, rows, N, ld, row0;
};

template <bool OUT_BF16>
__device__ __forceinline__ void splitk_reduce_body(const ReduceArgs& a) {
  const int chunks = (a.N + 7) / 8;
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(a.rows) * chunks) return;
  const int r = int(idx / chunks);
  const int n = int(idx - int64_t(r) * chunks) * 8;
  const bool hi = n + 4 < a.N;                     // second vector inside the row
  const size_t plane = (size_t)a.rows * a.ld;
  const float* src = a.ws + (size_t)r * a.ld + n;
  float4 x0 = *reinterpret_cast<const float4*>(src);
  float4 x1 = hi ? *reinterpret_cast<const float4*>(src + 4) : float4{0.f, 0.f, 0.f, 0.f};
  for (int s = 1; s < a.splits; ++s) {
    const float* t = src + s * plane;
    const float4 y0 = *reinterpret_cast<const float4*>(t);
    x0.x += y0.x; x0.y += y0.y; x0.z += y0.z; x0.w += y0.w;
    if (hi) {
      const float4 y1 = *reinterpret_cast<const float4*>(t + 4);
      x1.x += y1.x; x1.y += y1.y; x1.z += y1.z; x1.w += y1.w;
    }
  }
  const float v[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  store_row_span<OUT_BF16, 8>(a.C, size_t(a.row0 + r) * a.N, n, a.N, v);
}

// Named kernels (one per tile shape and output type) around the body.
// One named kernel per tile shape, output type and pair of operand formats
// (suffix _a<A format>b<B format>, 4 = E4M3, 5 = E5M2; E4M3 x E4M3 keeps the
// plain name); suffix _rs: row-scaled A (1 x 128 scales).
#define DG_GEMM_KERNEL_DEF(NAME, NWM, NWN, WN, BF16, FA, FB, RS)            \
  __global__ __launch_bounds__(64 * NWM * NWN, 1) void NAME(GemmArgs p) {   \
    gemm_f16mma_body<NWM, NWN, BF16, FA, FB, RS, WN>(p);                    \
  }
#define DG_GEMM_KERNEL_DECL(NAME, NWM, NWN, WN, BF16, FA, FB, RS) \
  __global__ __launch_bounds__(64 * NWM * NWN, 1) void NAME(GemmArgs p);
#define DG_GEMM_SHAPE(K, SHAPE, NWM, NWN, WN, SFX, FA, FB, RS)              \
  K(dg_gemm_##SHAPE##_bf16##SFX, NWM, NWN, WN, true, FA, FB, RS)            \
  K(dg_gemm_##SHAPE##_f32##SFX, NWM, NWN, WN, false, FA, FB, RS)
#define DG_GEMM_FORMATS(K, SFX, FA, FB)                                     \
  DG_GEMM_SHAPE(K, 128x512, 2, 4, 128, SFX, FA, FB, false)                  \
  DG_GEMM_SHAPE(K, 128x256, 2, 2, 128, SFX, FA, FB, false)                  \
  DG_GEMM_SHAPE(K, 128x256w8, 2, 4, 64, SFX, FA, FB, false)                 \
  DG_GEMM_SHAPE(K, 128x128w4, 2, 2, 64, SFX, FA, FB, false)                 \
  DG_GEMM_SHAPE(K, 128x64w2, 2, 1, 64, SFX, FA, FB, false)                  \
  DG_GEMM_SHAPE(K, 128x512, 2, 4, 128, SFX##_rs, FA, FB, true)              \
  DG_GEMM_SHAPE(K, 128x256, 2, 2, 128, SFX##_rs, FA, FB, true)              \
  DG_GEMM_SHAPE(K, 128x256w8, 2, 4, 64, SFX##_rs, FA, FB, true)             \
  DG_GEMM_SHAPE(K, 128x128w4, 2, 2, 64, SFX##_rs, FA, FB, true)             \
  DG_GEMM_SHAPE(K, 128x64w2, 2, 1, 64, SFX##_rs, FA, FB, true)
DG_GEMM_FORMATS(DG_KERNEL(DG_GEMM_KERNEL, FMT_44), , FMT_E4M3, FMT_E4M3)
DG_GEMM_FORMATS(DG_KERNEL(DG_GEMM_KERNEL, FMT_55), _a5b5, FMT_E5M2, FMT_E5M2)
DG_GEMM_FORMATS(DG_KERNEL(DG_GEMM_KERNEL, FMT_45), _a4b5, FMT_E4M3, FMT_E5M2)
DG_GEMM_FORMATS(DG_KERNEL(DG_GEMM_KERNEL, FMT_54), _a5b4, FMT_E5M2, FMT_E4M3)
#undef DG_GEMM_FORMATS
#undef DG_GEMM_SHAPE
#undef DG_GEMM_KERNEL_DECL
#undef DG_GEMM_KERNEL_DEF

#define DG_REDUCE_KERNEL_DEF(NAME, BF16) \
  __global__ __launch_bounds__(256) void NAME(ReduceArgs a) { splitk_reduce_body<BF16>(a); }
#define DG_REDUCE_KERNEL_DECL(NAME, BF16) __global__ __launch_bounds__(256) void NAME(ReduceArgs a);
DG_KERNEL(DG_REDUCE_KERNEL, MISC)(dg_splitk_reduce_bf16, true)
DG_KERNEL(DG_REDUCE_KERNEL, MISC)(dg_splitk_reduce_f32, false)
#undef DG_REDUCE_KERNEL_DECL
#undef DG_REDUCE_KERNEL_DEF

}  // namespace dg
