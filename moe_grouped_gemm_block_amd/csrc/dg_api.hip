// Host side of libdg.so: argument checks, kernel choice and launch.
//
// Every check that can be made without touching the device happens here,
// before any HIP call, so that argument errors are reported synchronously
// and the same checks run on a machine without a GPU.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "dg.h"
// this translation unit defines the quantiser; the GEMM kernels of each
// operand-format pair are defined in kernels_*.hip
#define DG_DEFINE_MISC
#include "gemm_f16mma.hpp"
#include "gemm_sharedb.hpp"
#include "gemm_skinny.hpp"
#include "quant.hpp"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
// Byte offsets inside a 512-row tile are 32-bit: 512 * K < 2^32.
constexpr int64_t kMaxK = int64_t(1) << 22;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shared checks of both entry points.  rows = M (dense) or M_total (grouped).
int check_common(const void* A, const float* sA, const void* B, const float* sB, void* C,
                 int64_t rows, int64_t N, int64_t K, int out_dtype) {
  if (rows < 0 || N < 0 || K < 0 || rows > kMaxDim || N > kMaxDim || K > kMaxDim)
    return DG_ERR_INVALID_ARG;
  if (out_dtype != DG_OUT_F32 && out_dtype != DG_OUT_BF16) return DG_ERR_INVALID_ARG;
  if (rows == 0 || N == 0) return DG_OK;
  if (C == nullptr || !aligned(C, 16)) return DG_ERR_INVALID_ARG;
  if (K > 0) {
    if (A == nullptr || B == nullptr || sA == nullptr || sB == nullptr) return DG_ERR_INVALID_ARG;
    if (!aligned(A, 16) || !aligned(B, 16) || !aligned(sA, 4) || !aligned(sB, 4))
      return DG_ERR_INVALID_ARG;
  }
  // rows of A and B must start 16-byte aligned (16-byte copies); the last
  // K-block may be partial, any N is fine
  if (K % 16 != 0) return DG_ERR_UNSUPPORTED;
  if (K > kMaxK) return DG_ERR_UNSUPPORTED;
  return DG_OK;
}

// Tile shape of one launch.  Dense problems whose 256 x 256 tiles fill whole
// rounds of the CUs (4096^3, 8192^2 x K, ...) run on the shared-B 256 x 256
// tile (gemm_sharedb.hpp: 8 waves of 32 x 256, B converted once per
// workgroup into LDS).  Otherwise the 128 x 512 tile runs 8 waves of 64 x 128
// (two per SIMD, one workgroup per CU, 160 KB of LDS).
// Narrow problems and the last partial round of a large one run on the
// narrow tiles chosen by launch_narrow: 128 x 256 (4 waves of 64 x 128 or 8
// of 64 x 64), 128 x 128 (4 waves of 64 x 64) or 128 x 64 (2 waves of
// 64 x 64).
// DG_FORCE_TILE=512 or 256 uses that tile for every problem (few rows
// included), 3256 the shared-B 256 x 256 tile for every dense problem, and
// 8256 /
// 4128 / 264 the 8-wave 128 x 256 / 4-wave 128 x 128 / 2-wave 128 x 64 tile
// wherever a narrow tile is used; DG_TAIL_TILE=0 / 256 / 8256 / 4128 / 264
// switches off the separate last round or sets the tile of narrow launches
// (256: launch_narrow's choice; the others as for DG_FORCE_TILE) (tuning
// aids).

// Compute units of the current device (one workgroup of the tiled kernels
// fills one), queried once per device and cached; 256 on the MI355X.
int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int forced_tile() {
  static const int v = [] {
    const char* e = getenv("DG_FORCE_TILE");
    return e ? atoi(e) : 0;
  }();
  return v;
}

int tail_tile() {
  static const int v = [] {
    const char* e = getenv("DG_TAIL_TILE");
    return e ? atoi(e) : 256;
  }();
  return v;
}

// DG_VALIDATE=1 (read once per process): grouped calls first copy
// group_offsets to the host, synchronising `stream`, and reject offsets that
// break the layout rules with DG_ERR_INVALID_ARG.  A debugging aid: the call
// is then no longer asynchronous and cannot be captured into a graph.
bool validate_offsets() {
  static const bool v = [] {
    const char* e = getenv("DG_VALIDATE");
    return e != nullptr && atoi(e) != 0;
  }();
  return v;
}

// 0 = o_0 <= o_1 <= ... <= o_G = M_total, and every o_e a multiple of 128
// when the segments are padded; with real row counts, 0 <= count_e <=
// o_{e+1} - o_e.
int check_offsets(const int32_t* offs, int G, int64_t M_total, bool padded, hipStream_t stream,
                  const int32_t* counts = nullptr) {
  if (!validate_offsets()) return DG_OK;
  std::vector<int32_t> h(size_t(G) + 1), c(counts ? size_t(G) : 0);
  if (hipMemcpyAsync(h.data(), offs, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      (counts && hipMemcpyAsync(c.data(), counts, c.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream) !=
                     hipSuccess) ||
      hipStreamSynchronize(stream) != hipSuccess)
    return DG_ERR_LAUNCH;
  if (h[0] != 0 || int64_t(h[size_t(G)]) != M_total) return DG_ERR_INVALID_ARG;
  for (int g = 0; g < G; ++g) {
    if (h[size_t(g) + 1] < h[size_t(g)]) return DG_ERR_INVALID_ARG;
    if (padded && h[size_t(g) + 1] % dg::KBLK != 0) return DG_ERR_INVALID_ARG;
    if (counts && (c[size_t(g)] < 0 || c[size_t(g)] > h[size_t(g) + 1] - h[size_t(g)])) return DG_ERR_INVALID_ARG;
  }
  return DG_OK;
}

// ---- split-K workspace -------------------------------------------------------
// A launch with fewer workgroups than CUs leaves the rest of the chip idle;
// splitting K over several copies of its tile grid fills it, at the price of
// writing FP32 partial tiles and adding them up in a second kernel (in a fixed
// order, so the result does not depend on scheduling).  The partials live in
// a workspace of kWsBytes per (device, stream), allocated by the first call
// on that stream that splits and kept until the process ends (a graph
// captured on the stream refers to it).  Calls on one stream are ordered, so
// they share it safely; calls on different streams use different
// workspaces.  A graph captured on a stream uses that stream's workspace
// when it is replayed: replays that overlap other calls made on the capture
// stream, or other replays of graphs captured on it, race.
// The allocation is made even while the stream is being captured (this
// thread's capture mode is switched to relaxed around hipMalloc, which
// enqueues nothing), so that a call computes the same result captured or
// not; only if the allocation fails does the call run unsplit.
constexpr size_t kWsBytes = size_t(32) << 20;

struct Workspace {
  int dev;
  hipStream_t stream;
  float* p;
};

float* stream_workspace(hipStream_t stream) {
  static std::mutex mu;
  static std::vector<Workspace> all;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  for (const Workspace& w : all)
    if (w.dev == dev && w.stream == stream) return w.p;
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) return nullptr;
  void* p = nullptr;
  const hipError_t err = hipMalloc(&p, kWsBytes);
  (void)hipThreadExchangeStreamCaptureMode(&mode);   // back to the caller's mode
  if (err != hipSuccess) {
    (void)hipGetLastError();   // leave no sticky error behind: the call runs unsplit
    return nullptr;
  }
  all.push_back({dev, stream, static_cast<float*>(p)});
  return static_cast<float*>(p);
}

// ---- the static scratch of dg_gemm_fp8_ex_noalloc ---------------------------
// For callers that cannot allocate: the split-K partials go to this array
// (one copy per device, loaded with the library's code object and held until
// the process ends) instead of a stream workspace.  Its size equals the
// stream workspace's, so both calls split alike and give the same bits.
// Every call on a device shares it: calls that overlap in time on one device
// race.  Nothing in it needs clearing: every partial is written before it is
// read.  In host code `scratch` is a stand-in for the device copy; kernels
// get the address from scratch_address().
constexpr size_t kScratchBytes = kWsBytes;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

// Device address of the current device's scratch, looked up once per device
// (with that device current) and cached; nullptr if the lookup fails.
float* scratch_address() {
  static std::mutex mu;
  static float* addr[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    addr[dev] = static_cast<float*>(p);
  }
  return addr[dev];
}

// DG_SPLITK (read once): unset or 0 = automatic, 1 = never split, S > 1 =
// split every launch of the tiled kernels into S parts (tuning aid).
int splitk_override() {
  static const int v = [] {
    const char* e = getenv("DG_SPLITK");
    return e ? atoi(e) : 0;
  }();
  return v;
}

// One launch over the row tiles [m_tile0, m_tile0 + m_tiles) of the kernel's
// tile height (128 rows unless stated; m_tiles < 0: all 128-row tiles).
// `splittable`: the kernels take a split of K (gemm_f16mma.hpp); the launch
// then splits K `splits` ways (DG_SPLITK > 1 overrides), fewer if the
// partials would not fit the workspace, none without a workspace.  The
// partials go to a.ws when the caller set it (the static scratch), else to
// the stream's workspace.
int launch_tiles(dg::GemmArgs a, int bn, int threads, void (*k_bf16)(dg::GemmArgs),
                 void (*k_f32)(dg::GemmArgs), int out_dtype, hipStream_t stream, int m_tile0 = 0,
                 int m_tiles = -1, bool splittable = true, int splits = 1) {
  a.m_tile0 = m_tile0;
  a.m_tiles = m_tiles >= 0 ? m_tiles : int((int64_t(a.M) + 127) / 128);
  a.n_tiles = int((int64_t(a.N) + bn - 1) / bn);
  a.splits = 1;
  const int64_t blocks = int64_t(a.m_tiles) * a.n_tiles;
  if (blocks <= 0) return DG_OK;
  if (blocks > INT32_MAX) return DG_ERR_UNSUPPORTED;
  const int64_t row0 = int64_t(m_tile0) * 128;
  const int64_t rows = std::min<int64_t>(int64_t(a.M) - row0, int64_t(a.m_tiles) * 128);
  int S = !splittable ? 1 : splitk_override() > 1 ? splitk_override() : splitk_override() == 1 ? 1 : splits;
  const int64_t plane = rows * ((int64_t(a.N) + 3) / 4 * 4) * 4;
  const bool preset = a.ws != nullptr;
  while (S > 1 && int64_t(S) * plane > int64_t(preset ? kScratchBytes : kWsBytes)) --S;
  if (S > 1 && !preset) {
    a.ws = stream_workspace(stream);
    if (a.ws == nullptr) S = 1;
  }
  if (S > 1 && (blocks * S > INT32_MAX || rows * ((int64_t(a.N) + 7) / 8) > INT32_MAX)) S = 1;
  if (S > 1) {
    a.splits = S;
    a.ws_ld = int((int64_t(a.N) + 3) / 4 * 4);
    a.ws_rows = int(rows);
  }
  void* kargs[] = {&a};
  const void* fn = out_dtype == DG_OUT_BF16 ? reinterpret_cast<const void*>(k_bf16)
                                            : reinterpret_cast<const void*>(k_f32);
  hipError_t err = hipLaunchKernel(fn, dim3(unsigned(blocks * S)), dim3(threads), kargs, 0, stream);
  if (err != hipSuccess) return DG_ERR_LAUNCH;
  if (S == 1) return DG_OK;
  dg::ReduceArgs r{a.ws, a.C, S, int(rows), a.N, a.ws_ld, int(row0)};
  const int64_t threads_r = rows * ((int64_t(a.N) + 7) / 8);
  void* rargs[] = {&r};
  const void* rfn = out_dtype == DG_OUT_BF16 ? reinterpret_cast<const void*>(dg::dg_splitk_reduce_bf16)
                                             : reinterpret_cast<const void*>(dg::dg_splitk_reduce_f32);
  err = hipLaunchKernel(rfn, dim3(unsigned((threads_r + 255) / 256)), dim3(256), rargs, 0, stream);
  return err == hipSuccess ? DG_OK : DG_ERR_LAUNCH;
}

typedef void (*kfn)(dg::GemmArgs);

// Kernels of one pair of operand formats; combo = 2 * a_fmt + b_fmt.  The
// *rs kernels take one A scale per row (1 x 128 blocks).
struct TiledSet { kfn sb256[2], k512[2], k256[2], k256w8[2], k128w4[2], k64w2[2]; };   // [f32, bf16]
#define DG_TILED_SET(SFX)                                                   \
  {{dg::dg_gemm_sb256_f32##SFX, dg::dg_gemm_sb256_bf16##SFX},               \
   {dg::dg_gemm_128x512_f32##SFX, dg::dg_gemm_128x512_bf16##SFX},           \
   {dg::dg_gemm_128x256_f32##SFX, dg::dg_gemm_128x256_bf16##SFX},           \
   {dg::dg_gemm_128x256w8_f32##SFX, dg::dg_gemm_128x256w8_bf16##SFX},       \
   {dg::dg_gemm_128x128w4_f32##SFX, dg::dg_gemm_128x128w4_bf16##SFX},       \
   {dg::dg_gemm_128x64w2_f32##SFX, dg::dg_gemm_128x64w2_bf16##SFX}}
// [A scales per 128 x 128 block / per row][combo]
const TiledSet kTiled[2][4] = {
    {DG_TILED_SET(), DG_TILED_SET(_a4b5), DG_TILED_SET(_a5b4), DG_TILED_SET(_a5b5)},
    {DG_TILED_SET(_rs), DG_TILED_SET(_a4b5_rs), DG_TILED_SET(_a5b4_rs), DG_TILED_SET(_a5b5_rs)}};
#undef DG_TILED_SET

// [A scales per block / per row][rows 16/32/64][NI 1/3][f32/bf16]
struct SkinnySet { kfn t[2][3][2][2]; };
#define DG_SKINNY_ROWS(SFX)                                                                                 \
  {{{dg::dg_skinny_m16_n16_f32##SFX, dg::dg_skinny_m16_n16_bf16##SFX},                                     \
    {dg::dg_skinny_m16_n48_f32##SFX, dg::dg_skinny_m16_n48_bf16##SFX}},                                    \
   {{dg::dg_skinny_m32_n16_f32##SFX, dg::dg_skinny_m32_n16_bf16##SFX},                                     \
    {dg::dg_skinny_m32_n48_f32##SFX, dg::dg_skinny_m32_n48_bf16##SFX}},                                    \
   {{dg::dg_skinny_m64_n16_f32##SFX, dg::dg_skinny_m64_n16_bf16##SFX},                                     \
    {dg::dg_skinny_m64_n48_f32##SFX, dg::dg_skinny_m64_n48_bf16##SFX}}}
#define DG_SKINNY_SET(SFX) {{DG_SKINNY_ROWS(SFX), DG_SKINNY_ROWS(SFX##_rs)}}
const SkinnySet kSkinny[4] = {DG_SKINNY_SET(), DG_SKINNY_SET(_a4b5), DG_SKINNY_SET(_a5b4), DG_SKINNY_SET(_a5b5)};
#undef DG_SKINNY_SET
#undef DG_SKINNY_ROWS

// Few rows (M <= 64, dense): one workgroup per 16*NI columns, its four waves
// splitting K; NI = 3 once that still gives every CU a workgroup.
int launch_skinny(dg::GemmArgs a, int out_dtype, int combo, int row_sa, hipStream_t stream) {
  const int rows = a.M <= 16 ? 0 : a.M <= 32 ? 1 : 2;
  const int wide = int64_t(a.N) >= int64_t(48) * num_cus() ? 1 : 0;
  const int cols = wide ? 48 : 16;
  const int64_t blocks = (int64_t(a.N) + cols - 1) / cols;
  if (blocks > INT32_MAX) return DG_ERR_UNSUPPORTED;
  void* kargs[] = {&a};
  const void* fn =
      reinterpret_cast<const void*>(kSkinny[combo].t[row_sa][rows][wide][out_dtype == DG_OUT_BF16 ? 1 : 0]);
  hipError_t err = hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(256), kargs, 0, stream);
  return err == hipSuccess ? DG_OK : DG_ERR_LAUNCH;
}

// Unpadded expert segments: [NI 1/3][f32/bf16]
struct SegSet { kfn t[2][2]; };
#define DG_SEG_SET(SFX)                                                     \
  {{{dg::dg_segments_n16_f32##SFX, dg::dg_segments_n16_bf16##SFX},          \
    {dg::dg_segments_n48_f32##SFX, dg::dg_segments_n48_bf16##SFX}}}
const SegSet kSeg[4] = {DG_SEG_SET(), DG_SEG_SET(_a4b5), DG_SEG_SET(_a5b4), DG_SEG_SET(_a5b5)};
#undef DG_SEG_SET

// One workgroup per (expert, column slab); the kernel picks the chunk height
// per expert.  The slab width is 48 once that still gives every CU a
// workgroup.
int launch_segments(dg::GemmArgs a, int out_dtype, int combo, hipStream_t stream) {
  const int wide = int64_t(a.G) * ((int64_t(a.N) + 47) / 48) >= num_cus() ? 1 : 0;
  const int cols = wide ? 48 : 16;
  const int64_t slabs = (int64_t(a.N) + cols - 1) / cols;
  const int64_t blocks = slabs * a.G;
  if (blocks > INT32_MAX) return DG_ERR_UNSUPPORTED;
  a.n_tiles = int(slabs);
  void* kargs[] = {&a};
  const void* fn = reinterpret_cast<const void*>(kSeg[combo].t[wide][out_dtype == DG_OUT_BF16 ? 1 : 0]);
  hipError_t err = hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(256), kargs, 0, stream);
  return err == hipSuccess ? DG_OK : DG_ERR_LAUNCH;
}

// Tiles of 128 rows and at most 256 columns.  A launch whose workgroups all
// run at once takes about one tile's time, so what counts is rounds of
// workgroups (one per CU) times the time of one tile.  Per-tile times
// relative to the 8-wave 128 x 512 tile, measured on the MI355X at
// K = 4096 with one workgroup per CU:
//   128 x 256,  4 waves of 64 x 128   0.74
//   128 x 256,  8 waves of 64 x 64    0.69 while at most 3/4 of the CUs are
//                                     busy, 0.78 beyond (the chip then runs
//                                     at its power limit, and this tile
//                                     converts 2 values per MFMA, not 1.5)
//   128 x 128,  4 waves of 64 x 64    0.40
//   128 x  64,  2 waves of 64 x 64    0.38
enum NarrowTile { kN256w4 = 0, kN256w8, kN128w4, kN64w2, kNarrowTiles };

struct NarrowShape {
  int cols;          // tile width
  double t;          // per-tile time relative to 128 x 512
  double t_crowded;  // the same once more than 3/4 of the CUs hold a tile
};
constexpr NarrowShape kNarrow[kNarrowTiles] = {
    {256, 0.74, 0.74}, {256, 0.69, 0.78}, {128, 0.40, 0.40}, {64, 0.38, 0.38}};

int64_t rounds(int64_t wgs) { return (wgs + num_cus() - 1) / num_cus(); }

// Estimated time of `rows` row tiles x N columns on narrow tile t.
double narrow_time(int t, int64_t rows, int64_t N) {
  const NarrowShape& n = kNarrow[t];
  const int64_t wgs = rows * ((N + n.cols - 1) / n.cols);
  return double(rounds(wgs)) * (wgs <= 3 * num_cus() / 4 ? n.t : n.t_crowded);
}

// The narrow tile with the least estimated time (ties go to the wider tile).
int best_narrow(int64_t rows, int64_t N, double* est = nullptr) {
  int best = kN256w4;
  for (int t = kN256w4 + 1; t < kNarrowTiles; ++t)
    if (narrow_time(t, rows, N) < narrow_time(best, rows, N)) best = t;
  if (est) *est = narrow_time(best, rows, N);
  return best;
}

// Splits of K for `rows` row tiles x N columns on the 128 x 128 tile: as
// many copies of its grid as fit whole into one round of the CUs, at most 8,
// each with at least 8 K-blocks (below that the partials' write-out and the
// separate sum, ~5 us per launch, cost more than the idle CUs).  Measured
// (MI355X, K = 4096, BF16 out, graph replay; best narrow tile unsplit ->
// split): 128 x 4096 35.4 -> 20.2 us (4 splits), 256 x 4096 35.4 -> 22.6 us
// (4), 512 x 4096 35.7 -> 29.9 us (2), 128 x 12288 35.9 -> ~28 us (2);
// 256 x 4096 x 1024 (8 K-blocks) 11.3 us unsplit, 15 us split 2 ways.
int narrow_splits(int64_t rows, int64_t N, int Kb) {
  const int64_t tiles = rows * ((N + 127) / 128);
  if (tiles <= 0) return 1;
  return int(std::max<int64_t>(1, std::min<int64_t>({int64_t(num_cus()) / tiles, int64_t(Kb / 8), int64_t(8)})));
}

// The row tiles [m_tile0, m_tile0 + m_tiles) (all when m_tiles < 0) on the
// narrow tile with the least estimated time (or the one an override names),
// or split over K on the 128 x 128 tile when that fills idle CUs.
int launch_narrow(const dg::GemmArgs& a, const TiledSet& ks, int out_dtype, hipStream_t stream, int m_tile0 = 0,
                  int m_tiles = -1) {
  const int64_t rows = m_tiles >= 0 ? m_tiles : (int64_t(a.M) + 127) / 128;
  const int Kb = int((int64_t(a.K) + dg::KBLK - 1) / dg::KBLK);
  const int S = forced_tile() == 0 && splitk_override() == 0 ? narrow_splits(rows, a.N, Kb) : 1;
  if (S > 1)
    return launch_tiles(a, 128, 256, ks.k128w4[1], ks.k128w4[0], out_dtype, stream, m_tile0, m_tiles, true, S);
  int t = best_narrow(rows, a.N);
  if (forced_tile() == 256) t = kN256w4;
  if (forced_tile() == 8256 || tail_tile() == 8256) t = kN256w8;
  if (forced_tile() == 4128 || tail_tile() == 4128) t = kN128w4;
  if (forced_tile() == 264 || tail_tile() == 264) t = kN64w2;
  switch (t) {
    case kN64w2: return launch_tiles(a, 64, 128, ks.k64w2[1], ks.k64w2[0], out_dtype, stream, m_tile0, m_tiles);
    case kN128w4: return launch_tiles(a, 128, 256, ks.k128w4[1], ks.k128w4[0], out_dtype, stream, m_tile0, m_tiles);
    case kN256w8: return launch_tiles(a, 256, 512, ks.k256w8[1], ks.k256w8[0], out_dtype, stream, m_tile0, m_tiles);
    default: return launch_tiles(a, 256, 256, ks.k256[1], ks.k256[0], out_dtype, stream, m_tile0, m_tiles);
  }
}

int launch(const dg::GemmArgs& a, int out_dtype, int a_fmt, int b_fmt, int row_sa, hipStream_t stream) {
  const int combo = 2 * a_fmt + b_fmt;
  const TiledSet& ks = kTiled[row_sa][combo];
  if (a.offs == nullptr && a.M <= 64 && forced_tile() == 0)
    return launch_skinny(a, out_dtype, combo, row_sa, stream);
  const int64_t m_tiles = (int64_t(a.M) + 127) / 128;
  const int64_t wide = m_tiles * ((int64_t(a.N) + 511) / 512);
  bool use512 = a.N > 256 && wide >= num_cus() / 2;
  if (use512 && wide < num_cus()) {
    // less than one round of 128 x 512 tiles: narrower tiles may fill more CUs
    double narrow = 0.0;
    best_narrow(m_tiles, a.N, &narrow);
    if (narrow < 1.0) use512 = false;
  }
  if (forced_tile() == 512) use512 = true;
  if (forced_tile() == 256) use512 = false;
  if (forced_tile() == 8256 || forced_tile() == 4128 || forced_tile() == 264) return launch_narrow(a, ks, out_dtype, stream);
  if (a.offs == nullptr) {
    const int64_t m256 = (int64_t(a.M) + 255) / 256, t256 = m256 * ((int64_t(a.N) + 255) / 256);
    // dense problems whose 256 x 256 tiles fill whole rounds of the CUs: the
    // tile whose eight waves share one FP16 copy of B
    if (forced_tile() == 3256 || (forced_tile() == 0 && a.M % 256 == 0 && t256 % num_cus() == 0))
      return launch_tiles(a, 256, 512, ks.sb256[1], ks.sb256[0], out_dtype, stream, 0, int(m256), false);
  }
  if (use512 && forced_tile() == 0 && tail_tile() != 0) {
    // A 128 x 512 tile takes about as long whether 1 or all 256 CUs are busy,
    // so a last round that is only partly filled costs almost a full round.
    // The row tiles that fill whole rounds go in one launch; the remaining
    // rows follow as narrower tiles, many more and each a fraction of the
    // work, in a second launch on the same stream (no workspace: every output
    // tile is still computed whole by one workgroup).
    const int64_t nt = (int64_t(a.N) + 511) / 512;
    const int64_t T = m_tiles * nt;
    const int64_t main_m = (T / num_cus()) * num_cus() / nt;
    if (T % num_cus() != 0 && main_m > 0 && main_m < m_tiles) {
      int st = launch_tiles(a, 512, 512, ks.k512[1], ks.k512[0], out_dtype, stream, 0, int(main_m));
      if (st != DG_OK) return st;
      const int rest = int(m_tiles - main_m);
      return launch_narrow(a, ks, out_dtype, stream, int(main_m), rest);
    }
  }
  if (use512) return launch_tiles(a, 512, 512, ks.k512[1], ks.k512[0], out_dtype, stream);
  return launch_narrow(a, ks, out_dtype, stream);
}

bool valid_fmt(int f) { return f == DG_FP8_E4M3 || f == DG_FP8_E5M2; }

// noalloc: split-K partials go to the static scratch (dg_gemm_fp8_ex_noalloc)
int gemm_impl(const void* A, int a_fmt, const float* sA, int sa_rows, const void* B, int b_fmt,
              const float* sB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype, hipStream_t stream,
              bool noalloc = false) {
  if (!valid_fmt(a_fmt) || !valid_fmt(b_fmt)) return DG_ERR_INVALID_ARG;
  if (sa_rows != 128 && sa_rows != 1) return DG_ERR_INVALID_ARG;
  int st = check_common(A, sA, B, sB, C, M, N, K, out_dtype);
  if (st != DG_OK || M == 0 || N == 0) return st;
  dg::GemmArgs a{};
  if (noalloc) {
    // The automatic split never needs more than (compute units) x 64 KB of
    // partials (S copies of at most CUs / S tiles of 128 x 128 FP32); only the
    // DG_SPLITK override can ask for more than the scratch holds, and such a
    // call is rejected here, before any launch.
    const int64_t ld = (N + 3) / 4 * 4;
    if (splitk_override() > 1 && int64_t(splitk_override()) * M * ld * 4 > int64_t(kScratchBytes))
      return DG_ERR_UNSUPPORTED;
    a.ws = scratch_address();
    if (a.ws == nullptr) return DG_ERR_LAUNCH;
  }
  a.A = static_cast<const uint8_t*>(A);
  a.sA = sA;
  a.B = static_cast<const uint8_t*>(B);
  a.sB = sB;
  a.C = C;
  a.offs = nullptr;
  a.G = 1;
  a.M = int(M);
  a.N = int(N);
  a.K = int(K);
  return launch(a, out_dtype, a_fmt, b_fmt, sa_rows == 1, stream);
}

// counts: per-expert real row counts (dg_grouped_gemm_fp8_ex_counts), or
// nullptr (every row of a segment is computed)
int grouped_impl(const void* A, int a_fmt, const float* sA, int sa_rows, const void* B, int b_fmt,
                 const float* sB, void* C, const int32_t* group_offsets, int num_groups, int64_t M_total,
                 int64_t N, int64_t K, int out_dtype, hipStream_t stream, const int32_t* counts = nullptr,
                 bool with_counts = false) {
  if (!valid_fmt(a_fmt) || !valid_fmt(b_fmt)) return DG_ERR_INVALID_ARG;
  if (sa_rows != 128 && sa_rows != 1) return DG_ERR_INVALID_ARG;
  if (num_groups < 1) return DG_ERR_INVALID_ARG;
  if (M_total < 0 || M_total % dg::KBLK != 0) return DG_ERR_INVALID_ARG;
  int st = check_common(A, sA, B, sB, C, M_total, N, K, out_dtype);
  if (st != DG_OK || M_total == 0 || N == 0) return st;
  if (group_offsets == nullptr || !aligned(group_offsets, 4)) return DG_ERR_INVALID_ARG;
  if (with_counts && (counts == nullptr || !aligned(counts, 4))) return DG_ERR_INVALID_ARG;
  st = check_offsets(group_offsets, num_groups, M_total, true, stream, counts);
  if (st != DG_OK) return st;
  dg::GemmArgs a{};
  a.counts = counts;
  a.A = static_cast<const uint8_t*>(A);
  a.sA = sA;
  a.B = static_cast<const uint8_t*>(B);
  a.sB = sB;
  a.C = C;
  a.offs = group_offsets;
  a.G = num_groups;
  a.M = int(M_total);
  a.N = int(N);
  a.K = int(K);
  return launch(a, out_dtype, a_fmt, b_fmt, sa_rows == 1, stream);
}

}  // namespace

extern "C" {

int dg_grouped_gemm_fp8_segments(const void* A, int a_fmt, const float* sA, const void* B, int b_fmt,
                                 const float* sB, void* C, const int32_t* group_offsets, int num_groups,
                                 int64_t M_total, int64_t N, int64_t K, int out_dtype, hipStream_t stream) {
  if (!valid_fmt(a_fmt) || !valid_fmt(b_fmt)) return DG_ERR_INVALID_ARG;
  if (num_groups < 1) return DG_ERR_INVALID_ARG;
  int st = check_common(A, sA, B, sB, C, M_total, N, K, out_dtype);
  if (st != DG_OK || M_total == 0 || N == 0) return st;
  if (group_offsets == nullptr || !aligned(group_offsets, 4)) return DG_ERR_INVALID_ARG;
  st = check_offsets(group_offsets, num_groups, M_total, false, stream);
  if (st != DG_OK) return st;
  dg::GemmArgs a{};
  a.A = static_cast<const uint8_t*>(A);
  a.sA = sA;
  a.B = static_cast<const uint8_t*>(B);
  a.sB = sB;
  a.C = C;
  a.offs = group_offsets;
  a.G = num_groups;
  a.M = int(M_total);
  a.N = int(N);
  a.K = int(K);
  return launch_segments(a, out_dtype, 2 * a_fmt + b_fmt, stream);
}

int dg_gemm_fp8_blockscaled(const void* A, const float* sA, const void* B, const float* sB,
                            void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                            hipStream_t stream) {
  return gemm_impl(A, DG_FP8_E4M3, sA, 128, B, DG_FP8_E4M3, sB, C, M, N, K, out_dtype, stream);
}

int dg_grouped_gemm_fp8(const void* A, const float* sA, const void* B, const float* sB, void* C,
                        const int32_t* group_offsets, int num_groups, int64_t M_total,
                        int64_t N, int64_t K, int out_dtype, hipStream_t stream) {
  return grouped_impl(A, DG_FP8_E4M3, sA, 128, B, DG_FP8_E4M3, sB, C, group_offsets, num_groups, M_total, N,
                      K, out_dtype, stream);
}

int dg_gemm_fp8_ex(const void* A, int a_fmt, const float* sA, int sa_rows, const void* B, int b_fmt,
                   const float* sB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                   hipStream_t stream) {
  return gemm_impl(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, M, N, K, out_dtype, stream);
}

int dg_gemm_fp8_ex_noalloc(const void* A, int a_fmt, const float* sA, int sa_rows, const void* B, int b_fmt,
                           const float* sB, void* C, int64_t M, int64_t N, int64_t K, int out_dtype,
                           hipStream_t stream) {
  return gemm_impl(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, M, N, K, out_dtype, stream, true);
}

int dg_grouped_gemm_fp8_ex(const void* A, int a_fmt, const float* sA, int sa_rows, const void* B, int b_fmt,
                           const float* sB, void* C, const int32_t* group_offsets, int num_groups,
                           int64_t M_total, int64_t N, int64_t K, int out_dtype, hipStream_t stream) {
  return grouped_impl(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, group_offsets, num_groups, M_total, N, K,
                      out_dtype, stream);
}

int dg_grouped_gemm_fp8_ex_counts(const void* A, int a_fmt, const float* sA, int sa_rows, const void* B,
                                  int b_fmt, const float* sB, void* C, const int32_t* group_offsets,
                                  const int32_t* group_counts, int num_groups, int64_t M_total, int64_t N,
                                  int64_t K, int out_dtype, hipStream_t stream) {
  return grouped_impl(A, a_fmt, sA, sa_rows, B, b_fmt, sB, C, group_offsets, num_groups, M_total, N, K,
                      out_dtype, stream, group_counts, true);
}

int dg_quantize_fp8_blockscaled(const void* X, int in_dtype, void* Q, float* S, int64_t M, int64_t K,
                                int block_rows, hipStream_t stream) {
  if (in_dtype != DG_IN_F32 && in_dtype != DG_IN_BF16) return DG_ERR_INVALID_ARG;
  if (block_rows != 1 && block_rows != 128) return DG_ERR_INVALID_ARG;
  if (M < 0 || K < 0 || M > kMaxDim || K > kMaxDim) return DG_ERR_INVALID_ARG;
  if (M == 0 || K == 0) return DG_OK;
  if (X == nullptr || Q == nullptr || S == nullptr) return DG_ERR_INVALID_ARG;
  if (!aligned(X, 16) || !aligned(Q, 16) || !aligned(S, 4)) return DG_ERR_INVALID_ARG;
  if (K % dg::KBLK != 0 || K > kMaxK) return DG_ERR_UNSUPPORTED;
  dg::QuantArgs a{X, static_cast<uint8_t*>(Q), S, int(M), int(K)};
  const int64_t Kb = K / dg::KBLK;
  // one workgroup per 128 x 128 block, or per 32 1 x 128 blocks
  const int64_t blocks = block_rows == 128 ? ((M + 127) / 128) * Kb : (M * Kb + 31) / 32;
  if (blocks > INT32_MAX) return DG_ERR_UNSUPPORTED;
  const bool bf16 = in_dtype == DG_IN_BF16;
  const void* fn = block_rows == 128
      ? (bf16 ? reinterpret_cast<const void*>(dg::dg_quant_128x128_bf16) : reinterpret_cast<const void*>(dg::dg_quant_128x128_f32))
      : (bf16 ? reinterpret_cast<const void*>(dg::dg_quant_1x128_bf16) : reinterpret_cast<const void*>(dg::dg_quant_1x128_f32));
  void* kargs[] = {&a};
  hipError_t err = hipLaunchKernel(fn, dim3(unsigned(blocks)), dim3(block_rows == 128 ? 1024 : 256), kargs, 0,
                                   stream);
  return err == hipSuccess ? DG_OK : DG_ERR_LAUNCH;
}

const char* dg_status_string(int status) {
  switch (status) {
    case DG_OK: return "DG_OK: success";
    case DG_ERR_INVALID_ARG: return "DG_ERR_INVALID_ARG: invalid argument (null, misaligned, negative or oversized)";
    case DG_ERR_UNSUPPORTED:
      return "DG_ERR_UNSUPPORTED: shape not supported (GEMM: K % 16 != 0 or K > 2^22; quantiser: K % 128 != 0; "
             "dg_gemm_fp8_ex_noalloc: split-K partials larger than its 32 MB static scratch)";
    case DG_ERR_LAUNCH: return "DG_ERR_LAUNCH: kernel launch failed";
    default: return "unknown dg_status";
  }
}

}  // extern "C"
