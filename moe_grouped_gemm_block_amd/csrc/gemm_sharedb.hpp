// FP8 block-scaled GEMM, dense, 256 x 256 tiles with the B tile shared by
// all eight waves as FP16 in LDS (gfx950).
//
// Same arithmetic as gemm_f16mma.hpp (block-wise scaling of the DeepGEMM
// FP8-for-MoE page, 2kiu.com/news/5461879, sections 2.1 and 3.3): per
// 128-wide K-block the exact FP8 products are summed on the FP16 matrix
// cores (every E4M3 / E5M2 value is exactly an FP16 value), and the block
// partial P is rescaled in FP32, acc = fma(fp32(sA * sB), P, acc).
//
// What changes is where the FP8 -> FP16 conversion happens.  The matrix
// core consumes FP16 operands, so every FP8 byte has to be converted once
// per register file that uses it; converting both operands inside every
// wave costs (rows + columns of the wave tile) conversions per K-block, which
// for 64 x 128 waves is 1.5 conversions per MFMA -- as much vector issue time
// as the matrix core needs for the MFMAs themselves.  Here:
//   * wave w owns rows [32 w, 32 w + 32) of the 256-row tile and all 256
//     columns (2 x 16 MFMA tiles of 16 x 16).  Its A rows are private: they
//     are loaded straight from global memory into registers (bounds-checked
//     buffer loads, rows past M and K positions past K read as zeros) and
//     converted there, 32 conversions per K-block;
//   * the B tile of a K-block (256 rows of 128 codes) is loaded by all eight
//     waves together (32 rows each, whole 128-byte lines), converted once,
//     and written to LDS as FP16 (64 KB); every wave then reads its MFMA
//     operands from there.  That is another 32 conversions per wave and
//     K-block: 0.5 conversions per MFMA instead of 1.5;
//   * two FP16 stages (128 KB of LDS): while the MFMAs of K-block kb read
//     stage kb % 2, the waves convert K-block kb + 1 into the other stage;
//     the operands of K-block kb + 1 (A) and kb + 2 (B) are loaded into
//     registers early in K-block kb, a whole K-block ahead of their use.
//     One barrier per K-block, placed before its last column tile: that
//     tile's MFMAs then overlap the reads of the next K-block's first B
//     operands and the conversion of its A, so a new K-block starts with
//     its operands in registers.  Every load is an ordinary,
//     compiler-visible buffer load, so the compiler counts its waits;
//   * the FP16 rows are 256 bytes (16 granules of 16 bytes); granule g of
//     row r sits at g ^ swzb(r % 16), which makes the operand reads free of
//     bank conflicts (see swzb);
//   * B rows are permuted on their way into LDS (brow_of_col) so that with
//     B as the MFMA's first operand each lane ends up holding runs of 8
//     consecutive output columns: every 16-byte store of the epilogue
//     writes whole 64-byte pieces of C rows;
//   * a wave's 32 rows lie inside one 128-row scale block and its columns
//     span two 128-column blocks: two factors per K-block, one per column
//     half (per-row A scales: one per row and column half).
// Tiles are ordered so that each XCD (own L2) works on a compact group of
// row and column tiles (tile_of).
#pragma once

#include "gemm_f16mma.hpp"

namespace dg {

// XOR applied to the granule index (0..15) of FP16 row r (r % 16 decides):
// f(r) = (r & 3) | (p(r >> 2) << 2), p = {0, 2, 3, 1}.
// A ds_read_b128 is served in four clocks of 16 lanes; within each half-wave
// the lanes {0-3, 12-15, 20-23, 24-27} share one clock and {4-7, 8-11,
// 16-19, 28-31} the other (measured on gfx950), and a clock is free of
// conflicts when its 16 lanes hit 16 distinct 16-byte positions modulo 256
// bytes, i.e. 16 distinct granules of a 256-byte row.  The operand read of
// lane (q = lane / 16, r = lane % 16) for k-step st takes granule
// (4 q + st) ^ f(r) of row r.  Within one clock, q = 0 pairs with rows
// S0 = {0-3, 12-15} and q = 1 with S1 = {4-11} (or the other way round), so
// the clock is conflict-free when f(S0) and f(S1) are each closed under
// XOR 4 and disjoint: f maps S0 onto {0..7} and S1 onto {8..15}.  Lanes
// 32-63 (q = 2, 3) XOR the granule with 8 on top and behave the same.
__device__ __forceinline__ int swzb(int r) {
  return (r & 3) | (((0x78 >> (2 * ((r >> 2) & 3))) & 3) << 2);
}

// LDS row of B tile column c (0..255): column c = 32 j + 8 q + 4 h + r goes
// to row 16 (2 j + h) + 4 q + r, i.e. row i = 4 q + r of MFMA column tile
// 2 j + h.  The MFMA result of tile ni gives lane (q, r16) rows 4 q .. 4 q + 3
// of the tile, so tiles 2 j and 2 j + 1 together give it the 8 consecutive
// columns 32 j + 8 q .. 32 j + 8 q + 7.
__device__ __forceinline__ int brow_of_col(int c) {
  return (c & ~31) | (((c >> 2) & 1) << 4) | (((c >> 3) & 3) << 2) | (c & 3);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over `bytes` bytes at `base` (loads past the end return
// zeros).  Both fields go through readfirstlane: the descriptor must live in
// scalar registers, or the compiler wraps every load in a loop over lanes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = (uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32))))) << 32) |
                     uint32_t(__builtin_amdgcn_readfirstlane(int(uint32_t(a))));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), 0, __builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// Buffer offset `off` (below 2^31) of a 16-byte piece at K position k: pushed
// to 2^31 or beyond, past every buffer, when k >= K, so that the load
// returns zeros.  Written without a select, which the compiler would turn
// into a branch around the load.
__device__ __forceinline__ uint32_t past_k(uint32_t off, int k, int K) {
  return off | (uint32_t(K - 1 - k) & kOutOfRange);
}

template <bool OUT_BF16, int FA = FMT_E4M3, int FB = FMT_E4M3, bool ROW_SA = false>
__device__ __forceinline__ void gemm_sharedb_body(const GemmArgs& p) {
  constexpr int NW = 8;                      // waves
  constexpr int WM = 32;                     // rows per wave
  constexpr int BM = NW * WM, BN = 256;      // workgroup tile
  constexpr int MI = 2, NI = BN / 16;        // 16 x 16 MFMA tiles per wave
  constexpr int ROWB = 2 * KBLK;             // bytes of one FP16 B row (one K-block)
  constexpr int STAGE = BN * ROWB;           // 64 KB
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_of<8>(blockIdx.x, p.m_tiles, p.n_tiles, tm, tn);
  const int m0 = (p.m_tile0 + tm) * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int Kb = (K + KBLK - 1) / KBLK;          // the last K-block may be partial
  const int Nb = (N + KBLK - 1) / KBLK;
  const int wm0 = m0 + wave * WM;                // first row of this wave

  // ---- scales (scalar loads through the constant address space) ----------
  typedef const __attribute__((address_space(4))) float cfloat;
  const int mb = min(wm0 / KBLK, (M - 1) / KBLK);
  const int nb0 = min(n0 / KBLK, Nb - 1), nb1 = min(n0 / KBLK + 1, Nb - 1);
  cfloat* sAr = (cfloat*)(p.sA + (ROW_SA ? 0 : (size_t)mb * Kb));
  cfloat* sB0 = (cfloat*)(p.sB + (size_t)nb0 * Kb);
  cfloat* sB1 = (cfloat*)(p.sB + (size_t)nb1 * Kb);

  // ---- operand loads -------------------------------------------------------
  const int q = lane >> 4, r16 = lane & 15;
  // A: the wave's rows; buffer ends at the matrix edge (rows past M read 0).
  const int a_rows = max(0, min(M - wm0, WM));
  const __amdgpu_buffer_rsrc_t rA = buffer_rsrc(p.A + (size_t)wm0 * K, a_rows * K);
  // lane (q, r16) holds K bytes [32 q, 32 q + 32) of rows 16 mi + r16 (the
  // K position is added per load)
  const uint32_t a_lane = uint32_t(r16 * K);
  // B: the tile's rows (columns of C); rows past N read 0.  Wave w loads
  // tile rows 32 w + 8 c + lr, 16 bytes at 16 lg, c = 0..3, where (lr, lg)
  // is a permutation of the lane's bits: lr = lane bits {0, 1, 4}, lg =
  // lane bits {5, 2, 3}.  Each load instruction still covers 8 whole rows;
  // the permutation is what makes the FP16 stores into LDS conflict-free
  // (see convert_b).
  const __amdgpu_buffer_rsrc_t rB = buffer_rsrc(p.B + (size_t)n0 * K, max(0, min(N - n0, BN)) * K);
  const int lr = (lane & 3) | ((lane >> 2) & 4), lg = ((lane >> 5) & 1) | ((lane >> 1) & 6);
  const uint32_t b_lane = uint32_t((wave * 32 + lr) * K);      // + K position per load

  u32x4 araw[MI][2], braw[4];
  // K-block kb of A / B into registers; a 16-byte piece past K reads zeros
  // (its offset is pushed past the buffer), so K-blocks past the end load
  // nothing and need no branch.
  auto load_a = [&](int kb) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = kb * KBLK + 32 * q + 16 * h;
        const uint32_t off = past_k(a_lane + uint32_t(mi * 16 * K + k), k, K);
        araw[mi][h] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rA, int(off), 0, 0));
      }
  };
  auto load_b = [&](int kb) {
    const int k = kb * KBLK + 16 * lg;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t off = past_k(b_lane + uint32_t(c * 8 * K + k), k, K);
      braw[c] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rB, int(off), 0, 0));
    }
  };

  // ---- B conversion: braw[c] -> FP16 stage ---------------------------------
  // Lane holds K codes [16 lg, 16 lg + 16) of tile row 32 w + 8 c + lr; they
  // become FP16 granules 2 lg and 2 lg + 1 of that column's LDS row
  // brow_of_col(32 w + 8 c + lr) = row0 + 4 c, whose swizzle is
  // swzb(4 c + lr % 4) = (lr % 4) | (p(c) << 2): the byte offset inside the
  // stage is row0 * 256 + 1024 c + 16 ((2 lg + h) ^ (lr % 4)), XOR 64 p(c).
  // A ds_write_b128 was measured to conflict when 8 consecutive lanes hit
  // fewer than 8 distinct 16-byte positions of a 128-byte window (lanes
  // 8k .. 8k+7 of one row wrote granules of one parity: 2-way, 8 extra
  // cycles per store); with the lane bits permuted as above, every group of
  // 8 consecutive lanes covers two rows whose swizzles differ in bit 0, and
  // the 16-lane and read-clock groupings stay conflict-free too.
  const int row0 = brow_of_col(wave * 32 + lr);
  const uint32_t wr_off[2] = {uint32_t(row0 * ROWB + 16 * ((2 * lg) ^ (lr & 3))),
                              uint32_t(row0 * ROWB + 16 * ((2 * lg + 1) ^ (lr & 3)))};
  auto convert_b = [&](int c, int stage) {
    constexpr int P = 0x78;                       // p = {0, 2, 3, 1}, 2 bits each
    const uint32_t x = uint32_t(64 * ((P >> (2 * c)) & 3));
    const u32x4 w = braw[c];
    uint32_t h[8];
    fp8x4_to_f16<FB>(w.x, h[0], h[1]);
    fp8x4_to_f16<FB>(w.y, h[2], h[3]);
    fp8x4_to_f16<FB>(w.z, h[4], h[5]);
    fp8x4_to_f16<FB>(w.w, h[6], h[7]);
    uint8_t* st = lds + stage * STAGE + 1024 * c;
    *reinterpret_cast<uint4*>(st + (wr_off[0] ^ x)) = uint4{h[0], h[1], h[2], h[3]};
    *reinterpret_cast<uint4*>(st + (wr_off[1] ^ x)) = uint4{h[4], h[5], h[6], h[7]};
  };

  // ---- operand reads from LDS ----------------------------------------------
  // Lane (q, r16) reads, for column tile ni and k-step st, granule
  // (4 q + st) ^ f(r16) of row 16 ni + r16: K values [32 q + 8 st, +8).
  const int fr = swzb(r16);
  int rd_off[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) rd_off[st] = r16 * ROWB + 16 * ((4 * q + st) ^ fr);
  auto read_b = [&](int stage, int ni, int st) -> v8h {
    return *reinterpret_cast<const v8h*>(lds + stage * STAGE + ni * 16 * ROWB + rd_off[st]);
  };

  // ---- per-row A scales (1 x 128 blocks) ------------------------------------
  const __amdgpu_buffer_rsrc_t rS = buffer_rsrc(p.sA + (size_t)wm0 * Kb, ROW_SA ? a_rows * Kb * 4 : 0);
  float sa_row[MI] = {0.f, 0.f};
  auto load_row_scales = [&](int kb) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      sa_row[mi] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(rS, int(uint32_t(((mi * 16 + r16) * Kb + kb) * 4)), 0, 0));
  };

  v4f acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // Operands of the K-block about to start: A converted, B of column tile 0
  // read from its stage.  Both are prepared during the last column tile of
  // the K-block before (prologue for K-block 0), so that the MFMAs of a new
  // K-block can issue right away.
  v8h af[MI][4];
  v8h bf[4];
  auto convert_a = [&](int st) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      af[mi][st] = fp8_operand<FA>(__builtin_bit_cast(int4, araw[mi][0]), __builtin_bit_cast(int4, araw[mi][1]), st);
  };

  // ---- prologue: B(0) -> stage 0; A(0) converted; B(1) in flight -----------
  if (Kb > 0) {
    load_b(0);
    load_a(0);
#pragma unroll
    for (int c = 0; c < 4; ++c) convert_b(c, 0);
    load_b(1);
    if constexpr (ROW_SA) load_row_scales(0);
  }
  __syncthreads();
  if (Kb > 0) {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      convert_a(st);
      bf[st] = read_b(0, 0, st);
    }
  }

  float sa_next = Kb > 0 && !ROW_SA ? float(sAr[0]) : 1.f;
  float sb0_next = Kb > 0 ? sB0[0] : 0.f, sb1_next = Kb > 0 ? sB1[0] : 0.f;
  // Partials of column tiles ni (part[ni & 1]); the partial of the last
  // column tile is rescaled during column tile 0 of the next K-block, with
  // the factors of its own K-block (s_last; zero before the first K-block).
  // With per-row A scales the two extra live factors would not fit the
  // register budget: there the last tile is rescaled at the end of its
  // K-block.
  constexpr bool kDeferLast = !ROW_SA;
  v4f part[2][MI];
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) part[1][mi] = v4f{0.f, 0.f, 0.f, 0.f};
  float s_last[MI] = {0.f, 0.f};
  for (int kb = 0; kb < Kb; ++kb) {
    const int stage = kSingleStage ? 0 : kb & 1;
    // this K-block's factors: [mi][column half]
    float s[MI][2];
    if constexpr (ROW_SA) {
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        s[mi][0] = sa_row[mi] * sb0_next;
        s[mi][1] = 0.f;                          // set at column tile NI / 2
      }
    } else {
      const float s0 = sa_next * sb0_next, s1 = sa_next * sb1_next;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        s[mi][0] = s0;
        s[mi][1] = s1;
      }
    }
    const float sb1_cur = sb1_next;
    {
      const int kn = min(kb + 1, Kb - 1);        // stays in bounds at the last K-block
      if constexpr (!ROW_SA) sa_next = sAr[kn];
      sb0_next = sB0[kn];
      sb1_next = sB1[kn];
    }

    // Column tile ni, k-step st: 2 MFMAs (row tiles mi = 0, 1) per B
    // operand; the B operands of tile ni + 1 are read into the registers the
    // MFMAs free, and the rescale of tile ni - 1 (for tile 0: the last tile
    // of the previous K-block; with per-row A scales that one is rescaled at
    // the end of its own K-block) runs between the MFMAs of tile ni.  Tile 0
    // issues the loads of A(kb + 1) (its registers were freed by the
    // conversion of A(kb)); tiles 1-4 convert B(kb + 1) into the other stage
    // (read by every wave during K-block kb - 1, which the barrier before
    // its last tile has closed; past the last K-block this writes zeros into
    // a stage nobody reads); tile 4 issues the loads of B(kb + 2).  The one
    // barrier of the K-block sits before tile 15: by then every wave has
    // read its last operands from this K-block's stage and written its part
    // of the next.  Tile 15 then reads the next K-block's tile-0 operands
    // from the other stage and converts A(kb + 1), k-step by k-step, into
    // the registers its own MFMAs free.  Scheduling barriers between the
    // tiles keep this order.
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      v4f* pc = part[ni & 1];
      if (ni == NI - 1) {
        if constexpr (!kSingleStage) __syncthreads();
      }
      if (ni == 0) load_a(kb + 1);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          pc[mi] = mfma16_f16(bf[st], af[mi][st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : pc[mi]);
        if (ni + 1 < NI) {
          bf[st] = read_b(stage, ni + 1, st);
        } else {
          convert_a(st);
          if constexpr (!kSingleStage) bf[st] = read_b(stage ^ 1, 0, st);
        }
      }
      if (ni > 0 || kDeferLast) {
        const v4f* pp = part[(ni - 1) & 1];
#pragma unroll
        for (int mi = 0; mi < MI; ++mi) {
          const float f = ni == 0 ? s_last[mi] : s[mi][(ni - 1) >= NI / 2];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[mi][(ni + NI - 1) % NI][r] = __builtin_fmaf(f, pp[mi][r], acc[mi][(ni + NI - 1) % NI][r]);
        }
      }
      if constexpr (ROW_SA) {
        // per-row factors of the second column half, then the next
        // K-block's row scales into the registers they came from
        if (ni == NI / 2) {
#pragma unroll
          for (int mi = 0; mi < MI; ++mi) s[mi][1] = sa_row[mi] * sb1_cur;
          load_row_scales(min(kb + 1, Kb - 1));
        }
      }
      if constexpr (!kSingleStage) {
        if (ni >= 1 && ni <= 4) convert_b(ni - 1, stage ^ 1);
        if (ni == 4) load_b(kb + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if constexpr (kDeferLast) {
        s_last[mi] = s[mi][1];
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          acc[mi][NI - 1][r] = __builtin_fmaf(s[mi][1], part[1][mi][r], acc[mi][NI - 1][r]);
      }
    }
    if constexpr (kSingleStage) {
      __syncthreads();                          // every wave is done with the stage
#pragma unroll
      for (int c = 0; c < 4; ++c) convert_b(c, 0);
      load_b(kb + 2);
      __syncthreads();
#pragma unroll
      for (int st = 0; st < 4; ++st) bf[st] = read_b(0, 0, st);
    }
  }
  if constexpr (kDeferLast) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc[mi][NI - 1][r] = __builtin_fmaf(s_last[mi], part[1][mi][r], acc[mi][NI - 1][r]);
  }

  // ---- epilogue: column tiles 2j and 2j+1 of a lane hold
  // C[m][n0 + 32 j + 8 q + 0 .. 7] -------------------------------------------
  const int lane_e = lane_id();
  const int q_e = lane_e >> 4, r16_e = lane_e & 15;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = wm0 + mi * 16 + r16_e;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < NI / 2; ++j) {
      float v[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = acc[mi][2 * j][r];
        v[4 + r] = acc[mi][2 * j + 1][r];
      }
      store_row_span<OUT_BF16, 8, true>(p.C, size_t(m) * N, n0 + 32 * j + 8 * q_e, N, v);
    }
  }
}

// Named kernels: dg_gemm_sb256_{bf16,f32}<format suffix><_rs>.
#define DG_SB_KERNEL_DEF(NAME, BF16, FA, FB, RS) \
  __global__ __launch_bounds__(512, 1) void NAME(GemmArgs p) { gemm_sharedb_body<BF16, FA, FB, RS>(p); }
#define DG_SB_KERNEL_DECL(NAME, BF16, FA, FB, RS) __global__ __launch_bounds__(512, 1) void NAME(GemmArgs p);
#define DG_SB_FORMATS(K, SFX, FA, FB)                       \
  K(dg_gemm_sb256_bf16##SFX, true, FA, FB, false)           \
  K(dg_gemm_sb256_f32##SFX, false, FA, FB, false)           \
  K(dg_gemm_sb256_bf16##SFX##_rs, true, FA, FB, true)       \
  K(dg_gemm_sb256_f32##SFX##_rs, false, FA, FB, true)
DG_SB_FORMATS(DG_KERNEL(DG_SB_KERNEL, FMT_44), , FMT_E4M3, FMT_E4M3)
DG_SB_FORMATS(DG_KERNEL(DG_SB_KERNEL, FMT_55), _a5b5, FMT_E5M2, FMT_E5M2)
DG_SB_FORMATS(DG_KERNEL(DG_SB_KERNEL, FMT_45), _a4b5, FMT_E4M3, FMT_E5M2)
DG_SB_FORMATS(DG_KERNEL(DG_SB_KERNEL, FMT_54), _a5b4, FMT_E5M2, FMT_E4M3)
#undef DG_SB_FORMATS
#undef DG_SB_KERNEL_DECL
#undef DG_SB_KERNEL_DEF

}  // namespace dg
