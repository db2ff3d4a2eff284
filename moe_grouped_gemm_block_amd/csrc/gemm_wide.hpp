// FP8 block-scaled GEMM, 128 x 512 tiles with one FP8 -> FP16 conversion per
// operand element per workgroup (dense and MoE-grouped), gfx950.
//
// Same arithmetic as gemm_f16mma.hpp (exact FP8 -> FP16 conversion, FP16
// MFMA partial per 128-wide K-block, FP32 rescale by fp32(sA * sB) of the
// block, FP32 accumulation; DeepGEMM FP8-for-MoE page, 2kiu.com/news/5461879,
// sections 2.1 and 3.3).  What changes is who converts what, because the
// vector work (conversion + rescale) and not the matrix cores limits that
// kernel:
//
//   * 8 waves side by side (1 x 8): wave w owns all 128 rows and the 64
//     columns [64 w, 64 w + 64) of the tile.  Its B rows are private: the
//     wave copies them with its own buffer->LDS loads into a private LDS
//     region and only waits on its own vmcnt; it converts them to FP16 once
//     per K-block and keeps them in registers (64 x 128 values), converting
//     the next block's B while its last A rows of the current block are
//     multiplied;
//   * the A tile (128 x 128) is shared by all waves: its FP8 bytes are copied
//     into LDS (two stages), every thread converts 32 of them per K-block
//     into an FP16 LDS tile (two buffers), and the waves read that tile
//     directly as MFMA operands.  The conversion of block kb+1 is spread over
//     the MFMA steps of block kb, so one barrier per K-block is enough;
//   * per wave and K-block: 8 row steps x 16 MFMAs (16x16x32 FP16), rescale
//     FMAs of the previous row step interleaved with the first MFMAs of the
//     next.  About 1.6 vector instructions per MFMA instead of ~2.7.
//
// Every asynchronous load of this kernel targets LDS; none writes registers.
#pragma once

#include "gemm_f16mma.hpp"

namespace dg {

// XOR swizzle of the 16-byte granules of an FP16 A-tile row (256 bytes).
// gfx950 serves a 128-bit LDS read in four clocks of 16 lanes each; within
// each half-wave, lanes {0-3, 12-15, 20-23, 24-27} share one clock and
// {4-7, 8-11, 16-19, 28-31} the other (measured with per-lane address
// patterns).  A clock is conflict-free when its 16 lanes hit 16 different
// granule positions modulo 256 bytes.  The operand reads of the MFMA loop
// (lane: row r16, granule 4 q + st) and the conversion stores (thread: row
// t/4, granules 4 (t%4) + i) both satisfy that with this linear map of the
// row's low four bits; the plain g ^ r map does not (2-way conflicts).
__device__ __forceinline__ int a16_swz(int r) {
  return (r & 3) ^ (((r >> 2) & 1) * 8) ^ (((r >> 3) & 1) * 12);
}

// Granule swizzle of the FP8 A staging tile (128-byte rows): granule g of
// row r sits at slot g ^ ((r >> 2) & 1).  The conversion reads (thread t:
// row t/4, granules 2 (t%4) + h) are then conflict-free under the same
// clock grouping.
__device__ __forceinline__ int a8_swz(int r) { return (r >> 2) & 1; }

constexpr int WIDE_NW = 8;                           // waves, side by side along N
constexpr int WIDE_B_WAVE = 64 * KBLK;               // 8 KB: one K-block of a wave's 64 B rows
constexpr int WIDE_B_BYTES = WIDE_NW * WIDE_B_WAVE;  // 64 KB, one stage
constexpr int WIDE_A8_BYTES = 128 * KBLK;            // 16 KB FP8 A tile, per stage
constexpr int WIDE_A16_BYTES = 128 * KBLK * 2;       // 32 KB FP16 A tile, per buffer
constexpr int WIDE_LDS = WIDE_B_BYTES + 2 * WIDE_A8_BYTES + 2 * WIDE_A16_BYTES;   // 160 KB
static_assert(WIDE_LDS <= 160 * 1024, "gfx950 LDS per workgroup");

template <bool OUT_BF16>
__device__ __forceinline__ void gemm_wide_body(const GemmArgs& p) {
  constexpr int NW = WIDE_NW;
  constexpr int BM = 128, WN = 64, BN = NW * WN; // tile 128 x 512, wave 128 x 64
  constexpr int MI = BM / 16, NI = WN / 16;      // 8 x 4 MFMA tiles per wave
  constexpr int B_CH = WN / 8;                   // B copy instructions per wave and K-block
  constexpr int A_CH = BM * KBLK / 1024 / NW;    // A copy instructions per wave and K-block (2)
  static_assert(B_CH == 8 && A_CH == 2, "copy counts assumed by the waits");
  // LDS: [B wave 0] ... [B wave 7] [A8 stage 0] [A8 stage 1] [A16 buf 0] [A16 buf 1]
  __shared__ __attribute__((aligned(16))) uint8_t lds[WIDE_LDS];
  uint8_t* const lds_a8 = lds + WIDE_B_BYTES;
  uint8_t* const lds_a16 = lds_a8 + 2 * WIDE_A8_BYTES;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int tm, tn;
  tile_of<8>(blockIdx.x, p.m_tiles, p.n_tiles, tm, tn);
  const int m0 = (p.m_tile0 + tm) * BM, n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int Kb = K / KBLK;
  const int Nb = (N + KBLK - 1) / KBLK;

  int e = 0;
  if (p.offs != nullptr) {
    e = find_group(p.offs, p.G, m0);
    if (e >= p.G) return;                        // uniform across the workgroup
  }
  const int wn0 = n0 + wave * WN;                // first column of this wave
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* sAr = (cfloat*)(p.sA + (size_t)(m0 / KBLK) * Kb);
  cfloat* sBr = (cfloat*)(p.sB + ((size_t)e * Nb + min(wn0 / KBLK, Nb - 1)) * Kb);
  const uint32_t lds_base = uint32_t(reinterpret_cast<uintptr_t>(static_cast<void*>(lds)));

  // ---- this wave's B rows: private buffer->LDS copies ----------------------
  // LDS row p = 16 ni + ii of the wave region holds wave row
  // 16 (ii / 4) + 4 ni + ii % 4, so that after the MFMA (B as first operand)
  // lane group q holds the 16 consecutive columns 16 q .. 16 q + 15.
  // Chunk c (LDS rows 8c .. 8c+7): lane L -> LDS row 8c + L/8, slot L%8,
  // granule (L%8) ^ f(row) with f(row) = (L/8) ^ (c & 1).
  const int brows = max(0, min(N - wn0, WN));
  const i32x4 rB = make_rsrc(p.B + ((size_t)e * N + max(min(wn0, N), 0)) * K, uint32_t(brows) * uint32_t(K));
  const int lr = lane >> 3;
  // (odd chunks use granule ^ 1, i.e. the even offset ^ 16: K is a multiple
  // of 128, so the row part never touches bit 4)
  const uint32_t b_lane_even = uint32_t((16 * (lane >> 5) + (lr & 3)) * K + (((lane & 7) ^ lr) * 16));
  const uint32_t lds_b_wave = __builtin_amdgcn_readfirstlane(lds_base + uint32_t(wave * WIDE_B_WAVE));
  auto issue_b = [&](int kb) {
    const uint32_t ev = opaque(b_lane_even + uint32_t(kb * KBLK));
    const uint32_t od = ev ^ 16u;
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int row = 32 * (c & 1) + 4 * (c >> 1);
      copy16_to_lds(rB, ((c & 1) ? od : ev) + uint32_t(row * K), lds_b_wave + uint32_t(c * 1024));
    }
  };

  // ---- A tile: FP8 bytes -> LDS stage, FP16 tile converted once per WG -----
  // Copy j of wave w fills LDS rows 8 (2w + j) .. +7 of the stage: lane L ->
  // row R = 8 (2w + j) + L/8, slot L%8, holding granule (L%8) ^ a8_swz(R).
  // Rows past M read as zeros (bounds of the buffer resource).
  const i32x4 rA = make_rsrc(p.A + (size_t)m0 * K, uint32_t(min(M - m0, BM)) * uint32_t(K));
  const int a8_row = 16 * wave + (lane >> 3);    // row of copy j = 0 (j = 1: + 8, same swizzle)
  const uint32_t a8_lane = uint32_t(a8_row * K + (((lane & 7) ^ a8_swz(a8_row)) * 16));
  const uint32_t lds_a8_wave = __builtin_amdgcn_readfirstlane(
      lds_base + uint32_t(WIDE_B_BYTES + wave * A_CH * 1024));
  auto issue_a8 = [&](int kb, int stage) {
    const uint32_t o = opaque(a8_lane + uint32_t(kb * KBLK));
    const uint32_t dst = lds_a8_wave + uint32_t(stage * WIDE_A8_BYTES);
    copy16_to_lds(rA, o, dst);
    copy16_to_lds(rA, o + uint32_t(8 * K), dst + 1024u);
  };
  // Thread t converts FP8 granules 2 (t%4) + h (h = 0, 1) of tile row t/4;
  // granule g yields FP16 granules 2g and 2g + 1, stored at slot
  // (FP16 granule) ^ a16_swz(row) of the row's 256 bytes.
  const int ar = tid >> 2, aj = tid & 3;
  const int a8_rd0 = ar * KBLK + (((2 * aj) ^ a8_swz(ar)) * 16);   // h = 1: ^ 16
  const int a16_wr0 = ar * 256 + (((4 * aj) ^ a16_swz(ar)) * 16); // FP16 granule 4aj + u: ^ (16 u)
  auto read_a8 = [&](const uint8_t* a8, int h) {
    return *reinterpret_cast<const int4*>(a8 + (a8_rd0 ^ (16 * h)));
  };
  auto write_a16 = [&](uint8_t* a16, int h, const int4& x) {
    uint32_t w[8];
    fp8x4_to_f16(uint32_t(x.x), w[0], w[1]);
    fp8x4_to_f16(uint32_t(x.y), w[2], w[3]);
    fp8x4_to_f16(uint32_t(x.z), w[4], w[5]);
    fp8x4_to_f16(uint32_t(x.w), w[6], w[7]);
    *reinterpret_cast<uint4*>(a16 + (a16_wr0 ^ (32 * h))) = uint4{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<uint4*>(a16 + (a16_wr0 ^ (32 * h + 16))) = uint4{w[4], w[5], w[6], w[7]};
  };

  v4f acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int q = lane >> 4, r16 = lane & 15;
  // B fragment reads (wave region): rows 16 ni + r16, FP8 bytes [32q, 32q+32);
  // the second granule is the first one ^ 1 (offset ^ 16).
  const int b_off0_init = r16 * KBLK + swz16(r16, 2 * q) * 16;
  // A fragment reads (FP16 tile): row 16 mi + r16, FP16 granule 4q + st, i.e.
  // the st = 0 offset ^ (16 st).
  const int a16_base_init = r16 * 256 + (((4 * q) ^ a16_swz(r16)) * 16);
  const uint8_t* const lb = lds + wave * WIDE_B_WAVE;

  v8h bh[NI][4];                                 // FP16 B of the current K-block
  if (Kb > 0) {
    issue_b(0);
    issue_a8(0, 0);
    issue_a8(min(1, Kb - 1), 1);
    wait_vmem_n<A_CH>();                         // B(0), A(0) landed (A(1) may not have)
    __syncthreads();                             // A8(0) of every wave visible
#pragma unroll
    for (int h = 0; h < 2; ++h) write_a16(lds_a16, h, read_a8(lds_a8, h));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const int4 y0 = *reinterpret_cast<const int4*>(lb + b_off0_init + ni * 16 * KBLK);
      const int4 y1 = *reinterpret_cast<const int4*>(lb + (b_off0_init ^ 16) + ni * 16 * KBLK);
      fp8x32_to_f16(y0, y1, bh[ni]);
    }
    wait_vmem();                                 // A(1) landed
    __syncthreads();                             // A16(0), A8(1) visible; B region read
  }

  float sa_next = Kb > 0 ? sAr[0] : 0.f, sb_next = Kb > 0 ? sBr[0] : 0.f;
  for (int kb = 0; kb < Kb; ++kb) {
    // The loop body is kept free of branches (one basic block, so the
    // register allocator never has to keep old and new values alive across a
    // join): prefetch indices are clamped to the last K-block instead.  The
    // fragment offsets are rebuilt from opaque copies each K-block so that
    // only their two bases stay live across the loop.
    const int b_off0 = int(opaque(uint32_t(b_off0_init)));
    const int b_off1 = b_off0 ^ 16;
    const int a16_base = int(opaque(uint32_t(a16_base_init)));
    const float s = sa_next * sb_next;
    sa_next = sAr[min(kb + 1, Kb - 1)];
    sb_next = sBr[min(kb + 1, Kb - 1)];
    // The B region was read (B(kb) converted) before the last barrier, and A8
    // stage kb&1 held A(kb), converted during the previous K-block.
    issue_b(min(kb + 1, Kb - 1));
    issue_a8(min(kb + 2, Kb - 1), kb & 1);
    const uint8_t* a16 = lds_a16 + (kb & 1) * WIDE_A16_BYTES;
    uint8_t* a16_next = lds_a16 + ((kb + 1) & 1) * WIDE_A16_BYTES;
    const uint8_t* a8_next = lds_a8 + ((kb + 1) & 1) * WIDE_A8_BYTES;

    v8h af[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) af[st] = *reinterpret_cast<const v8h*>(a16 + (a16_base ^ (16 * st)));
    v4f part[NI];
    int4 xa;                                     // FP8 A granule between its read and its conversion
    uint2 yb[NI];                                // raw FP8 B of one next-block operand, read a group ahead
    // next block's B operand st of this lane: FP8 bytes 8 st .. 8 st + 7 of
    // its 32-byte slice, i.e. half st & 1 of granule st >> 1
    auto read_b8 = [&](int st) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        yb[ni] = *reinterpret_cast<const uint2*>(lb + ((st >> 1) ? b_off1 : b_off0) + 8 * (st & 1) + ni * 16 * KBLK);
    };
    // The body is a sequence of (row step mi, K sub-step st) groups separated
    // by scheduling fences: each group holds its 4 MFMAs, the rescale FMAs of
    // the previous row step (st = 0), the LDS read of the next row step's
    // operand st (one full step of latency before its use) and its share of
    // the A / B conversion work.  Inside a group the scheduler interleaves.
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          if (st == 0 && mi > 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[mi - 1][ni][r] = __builtin_fmaf(s, part[ni][r], acc[mi - 1][ni][r]);
          }
          part[ni] = mfma16_f16(bh[ni][st], af[st], st == 0 ? v4f{0.f, 0.f, 0.f, 0.f} : part[ni]);
        }
        if (mi + 1 < MI) {
          af[st] = *reinterpret_cast<const v8h*>(a16 + (mi + 1) * 16 * 256 + (a16_base ^ (16 * st)));
        } else {
          // operand st of the next K-block's B, converted into the registers
          // the MFMAs above have just consumed (unconditionally: on the last
          // K-block this converts data that is never used, which keeps the
          // old and new B values from both being live); its raw bytes were
          // read one group earlier, the next operand's are read now
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            uint32_t hh[4];
            fp8x4_to_f16(yb[ni].x, hh[0], hh[1]);
            fp8x4_to_f16(yb[ni].y, hh[2], hh[3]);
            bh[ni][st] = __builtin_bit_cast(v8h, (uint4{hh[0], hh[1], hh[2], hh[3]}));
          }
          if (st < 3) read_b8(st + 1);
        }
        if (mi == MI - 2 && st == 3) {
          wait_vmem_n<A_CH>();                   // B(kb+1) landed (A(kb+2) may not have)
          read_b8(0);
        }
        // A(kb+1): FP8 granule h read in step 1 + 2h, converted and stored in
        // step 2 + 2h
        if ((mi == 1 || mi == 3) && st == 1) xa = read_a8(a8_next, mi >> 1);
        if ((mi == 2 || mi == 4) && st == 2) write_a16(a16_next, (mi - 2) >> 1, xa);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[MI - 1][ni][r] = __builtin_fmaf(s, part[ni][r], acc[MI - 1][ni][r]);

    wait_vmem();                                 // A(kb+2) landed
    __syncthreads();                             // A16(kb+1), A8(kb+2) visible; A16(kb), B region read
  }

  // ---- epilogue: lane holds C[m][wn0 + 16 q + 0 .. 15] ------------------------
  const int lane_e = lane_id();
  const int q_e = lane_e >> 4, r16_e = lane_e & 15;
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int m = m0 + mi * 16 + r16_e;
    if (m >= M) continue;
    const int nbase = wn0 + 16 * q_e;
    float v[16];
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
#pragma unroll
      for (int r = 0; r < 4; ++r) v[ni * 4 + r] = acc[mi][ni][r];
    if constexpr (OUT_BF16) {
      uint16_t* row = reinterpret_cast<uint16_t*>(p.C) + (size_t)m * N;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int n = nbase + 8 * c;
        if (n >= N) continue;
        uint4 w;
        w.x = pack_bf16x2(v[8 * c + 0], v[8 * c + 1]);
        w.y = pack_bf16x2(v[8 * c + 2], v[8 * c + 3]);
        w.z = pack_bf16x2(v[8 * c + 4], v[8 * c + 5]);
        w.w = pack_bf16x2(v[8 * c + 6], v[8 * c + 7]);
        *reinterpret_cast<uint4*>(row + n) = w;
      }
    } else {
      float* row = reinterpret_cast<float*>(p.C) + (size_t)m * N;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int n = nbase + 4 * c;
        if (n >= N) continue;
        *reinterpret_cast<float4*>(row + n) = float4{v[4 * c], v[4 * c + 1], v[4 * c + 2], v[4 * c + 3]};
      }
    }
  }
}

#define DG_WIDE_KERNEL_DEF(NAME, BF16) \
  __global__ __launch_bounds__(512, 1) void NAME(GemmArgs p) { gemm_wide_body<BF16>(p); }
#define DG_WIDE_KERNEL_DECL(NAME, BF16) __global__ __launch_bounds__(512, 1) void NAME(GemmArgs p);
DG_KERNEL(DG_WIDE_KERNEL, MISC)(dg_gemm_wide_128x512_bf16, true)
DG_KERNEL(DG_WIDE_KERNEL, MISC)(dg_gemm_wide_128x512_f32, false)
#undef DG_WIDE_KERNEL_DECL
#undef DG_WIDE_KERNEL_DEF

}  // namespace dg
