/*
 * dg.h -- C ABI of libdg.so: block-scaled FP8 GEMM on AMD Instinct MI355X
 * (gfx950), dense and MoE-grouped, and the FP8 quantisation of activations
 * that produces its A operand.  The base calls take E4M3 operands with
 * 128x128 block scales; the _ex calls add E5M2 operands and per-token (1 x 128)
 * A scales, dg_grouped_gemm_fp8_segments serves decode-time MoE.
 *
 * The operation (DeepGEMM FP8-for-MoE page, 2kiu.com/news/5461879,
 * section 2.1 "block-wise scaling"; FP32 accumulation, section 3.3):
 *
 *   C[i][j] = sum over K-blocks kb of
 *             fp32(sA[i/128][kb] * sB[j/128][kb]) * P_kb[i][j],
 *   P_kb[i][j] = sum_{k = 128 kb}^{128 kb + 127} dec(A[i][k]) * dec(B[j][k])
 *
 * i.e. every 128-wide K-block's partial product is formed with FP32-grade
 * accumulation (on gfx950 by the FP16 matrix cores, which represent every
 * E4M3 value exactly) and then rescaled in FP32 by that block's A and B scale
 * factors before it is added to the FP32 accumulator.  dec() is the
 * OCP E4M3FN decode: 1 sign, 4 exponent (bias 7), 3 mantissa bits, largest
 * finite value 448 (DeepGEMM FP8 kernel write-up, demingchina.com/news/60142,
 * section 3.1 table).  The result is written once, as FP32 or as BF16
 * (round to nearest even).
 *
 * Layout (the caller supplies A, B and both scale sets; A row-major, B
 * column-major -- FP8-for-MoE page, section 4.3):
 *   A  : E4M3 bytes, [M][K] row-major (K contiguous)
 *   B  : E4M3 bytes, [N][K] row-major, i.e. the K x N operand stored
 *        column-major (K contiguous)
 *   sA : float32 [ceil(M/128)][Kb] row-major, Kb = ceil(K/128)
 *   sB : float32 [ceil(N/128)][Kb] row-major
 *   C  : [M][N] row-major, float32 or bfloat16 (out_dtype)
 *
 * Conventions shared by every entry point:
 *   - All data pointers are device memory owned by the caller.  The only
 *     memory the library allocates is the split-K workspace (next item);
 *     there is no other per-call state: calls are thread-safe and may run
 *     concurrently on different streams.
 *   - Split K.  A GEMM whose 128-row output tiles would occupy at most half
 *     of the GPU's compute units, with at least 16 K-blocks, is computed as S
 *     (2..8) partial GEMMs over consecutive ranges of K-blocks, each summed
 *     and rescaled per K-block exactly as above into FP32, then added in the
 *     order of their ranges: C = sum_s (sum_{kb in range s} fp32(sA sB) P_kb),
 *     one rounding to out_dtype at the end.  The FP32 partials live in a
 *     workspace of 32 MB per (device, stream), allocated by the first call
 *     on that stream that splits (also while the stream is being captured
 *     into a graph: the allocation is made in relaxed capture mode and
 *     enqueues nothing) and kept until the process ends.  Calls on one
 *     stream share it in stream order; calls on different streams use
 *     different workspaces.  A graph captured on a stream uses that
 *     stream's workspace whenever it is replayed: replays must not overlap
 *     other calls made on the capture stream or other replays of graphs
 *     captured on it.  If the allocation fails the call runs unsplit.
 *   - Calls are asynchronous: the work is enqueued on `stream` (0 = the null
 *     stream) and the call returns without synchronising.  Passing the stream
 *     explicitly lets a caller order the GEMM against collectives on the same
 *     stream (a race of that kind is discussed on the vLLM integration page,
 *     mpbf.cn/news/61361, section 5.5).
 *   - Argument errors are detected on the host before any HIP call and return
 *     DG_ERR_INVALID_ARG: a null pointer for a non-empty operand, negative or
 *     too large sizes (each of M, N, K must be below 2^31), an unknown
 *     out_dtype, A / B / C not 16-byte aligned, sA / sB / group_offsets not
 *     4-byte aligned.
 *   - Shapes outside the supported set return DG_ERR_UNSUPPORTED: K must be a
 *     multiple of 16 (so that every row of A and B starts 16-byte aligned)
 *     and at most 2^22.  M and N are arbitrary.
 *   - Kb = ceil(K/128) K-blocks.  When K is not a multiple of 128 the last
 *     K-block is partial: its P_kb sums the K - 128 (Kb - 1) remaining
 *     columns and its scales are those of that partial block (the scale
 *     arrays have Kb columns).
 *   - Empty work (M == 0 or N == 0) is a no-op that returns DG_OK.  K == 0
 *     writes zeros.
 *   - A failed kernel launch returns DG_ERR_LAUNCH.  Faults inside a kernel
 *     surface at the caller's next synchronisation, as for any HIP kernel.
 *   - Every call only enqueues kernels (no memset, no host synchronisation;
 *     apart from the workspace allocation above), so it may be captured into
 *     a HIP graph and replayed (the DG_VALIDATE=1 debugging aid of the
 *     grouped calls excepted).
 *   - Results are bitwise repeatable: no atomics, and every output element
 *     is summed in a fixed order (the split of K depends only on the shape
 *     and the GPU's compute unit count).
 *   - Out of scope: alpha / beta (C is overwritten, alpha = 1, beta = 0),
 *     transposed layouts other than the above, other element types.
 */
#ifndef DG_H_
#define DG_H_

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  DG_OUT_F32 = 0,   /* C is float32 */
  DG_OUT_BF16 = 1   /* C is bfloat16, rounded to nearest even from FP32 */
} dg_out_dtype;

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = -1,
  DG_ERR_UNSUPPORTED = -2,
  DG_ERR_LAUNCH = -3
} dg_status;

/*
 * Dense block-scaled FP8 GEMM, C = A x B with 128x128 block scales
 * (FP8-for-MoE page, section 2.1).  Shapes and layouts as above.
 */
int dg_gemm_fp8_blockscaled(const void* A, const float* sA,
                            const void* B, const float* sB,
                            void* C, int64_t M, int64_t N, int64_t K,
                            int out_dtype, hipStream_t stream);

/*
 * MoE grouped block-scaled FP8 GEMM in one launch over contiguous per-expert
 * row segments (the one-matrix expert layout of the shape-specialised-kernels
 * page, nxmr.cn/news/132300, section 2.2; MoE experts share N and K while
 * the row count varies, FP8-for-MoE page, section 2.2).
 *
 *   A             : E4M3 [M_total][K]; rows [o_e, o_{e+1}) belong to expert e
 *   sA            : float32 [M_total/128][Kb]
 *   B             : E4M3 [num_groups][N][K] (expert e's B_e, K contiguous)
 *   sB            : float32 [num_groups][ceil(N/128)][Kb]
 *   C             : [M_total][N] float32 or bfloat16
 *   group_offsets : DEVICE int32 [num_groups + 1] with
 *                   0 = o_0 <= o_1 <= ... <= o_G = M_total, every o_e a
 *                   multiple of 128 (segments are padded to 128 rows, so a
 *                   128-row tile or an A scale block never mixes experts).
 *                   Empty experts (o_e == o_{e+1}) are allowed.
 *
 * Rows of a segment that the caller padded with zero codes come out as
 * exact zeros.  The offsets live on the device and are not validated by
 * default (that needs a device-to-host synchronisation): offsets that break
 * the rules above give undefined values in C, but every access stays inside
 * A, B, sA, sB and C (a tile's expert is found by a bounded binary search
 * over the offsets).  Host-side errors: num_groups < 1 or M_total not a
 * multiple of 128 -> DG_ERR_INVALID_ARG; the shared rules above otherwise.
 *
 * Debugging aid: with the environment variable DG_VALIDATE=1 (read once per
 * process) the grouped calls first copy group_offsets to the host,
 * synchronising `stream`, and return DG_ERR_INVALID_ARG for offsets that
 * break the rules (DG_ERR_LAUNCH if that copy fails).  Such calls are no
 * longer asynchronous and cannot be captured into a HIP graph.
 */
int dg_grouped_gemm_fp8(const void* A, const float* sA,
                        const void* B, const float* sB,
                        void* C, const int32_t* group_offsets,
                        int num_groups, int64_t M_total, int64_t N, int64_t K,
                        int out_dtype, hipStream_t stream);

typedef enum {
  DG_FP8_E4M3 = 0,  /* OCP E4M3FN: bias 7, largest finite 448, no infinities */
  DG_FP8_E5M2 = 1   /* E5M2: bias 15, largest finite 57344, IEEE-style inf/NaN */
} dg_fp8_format;

/*
 * The two GEMMs above, generalised in two ways:
 *
 *   a_fmt, b_fmt : the code format of each operand (E4M3 and E5M2, the two
 *                  FP8 formats of the DeepGEMM FP8 kernel write-up's section
 *                  3.1 table; the FP8-for-MoE page, section 2.1, names both).
 *                  dec() of an operand is the decode of its format.  E5M2
 *                  values span 2^-16 .. 57344 and, like E4M3, are exact FP16
 *                  values, so the precision statement is unchanged; E5M2
 *                  infinity and NaN codes propagate.
 *   sa_rows      : rows per A scale block, 128 or 1.  128 is the 128 x 128
 *                  layout above.  1 gives every row (token) its own scale per
 *                  128-wide K-block, the 1 x 128 granularity of the FP8 kernel
 *                  write-up's section 5.2 table, which
 *                  dg_quantize_fp8_blockscaled(block_rows = 1) produces:
 *                    sA : float32 [M][Kb] row-major (grouped: [M_total][Kb])
 *                  and C[i][j] takes fp32(sA[i][kb] * sB[j/128][kb]) as the
 *                  factor of P_kb[i][j].  B keeps its 128 x 128 blocks.
 *
 * Everything else -- layouts, per-K-block FP32 rescale, FP32 accumulation,
 * output, errors -- is as documented for dg_gemm_fp8_blockscaled and
 * dg_grouped_gemm_fp8, which are these calls with a_fmt = b_fmt =
 * DG_FP8_E4M3 and sa_rows = 128.  An unknown format or an sa_rows other than
 * 1 or 128 is DG_ERR_INVALID_ARG.
 */
int dg_gemm_fp8_ex(const void* A, int a_fmt, const float* sA, int sa_rows,
                   const void* B, int b_fmt, const float* sB,
                   void* C, int64_t M, int64_t N, int64_t K,
                   int out_dtype, hipStream_t stream);

/*
 * dg_gemm_fp8_ex for callers that cannot allocate device memory: code under
 * HIP graph capture that must not allocate, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, layouts, result (bit for bit, when
 * dg_gemm_fp8_ex has its workspace: the same kernels and the same split of K)
 * and errors as dg_gemm_fp8_ex, except where the split-K partials go: a
 * static device buffer of 32 MB that the library holds on every device it
 * runs on until the process ends, instead of the per-stream workspace.  The
 * call allocates nothing (no hipMalloc, no allocating library routine); the
 * caller still provides A, B, the scales and C.
 *
 * The automatic split never needs more than 64 KB per compute unit of the
 * GPU (16 MB on the MI355X); a call whose partials would exceed the buffer
 * -- only the DG_SPLITK tuning override can ask for that -- returns
 * DG_ERR_UNSUPPORTED before any launch.  DG_ERR_LAUNCH if the buffer's
 * device address cannot be looked up.  Every call on a device shares that
 * device's buffer, which keeps the last call's contents (nothing in it needs
 * clearing: every partial is written before it is read): calls that overlap
 * in time on one device -- on different streams, or replays of captured
 * graphs -- race and give undefined results.
 */
int dg_gemm_fp8_ex_noalloc(const void* A, int a_fmt, const float* sA, int sa_rows,
                           const void* B, int b_fmt, const float* sB,
                           void* C, int64_t M, int64_t N, int64_t K,
                           int out_dtype, hipStream_t stream);

int dg_grouped_gemm_fp8_ex(const void* A, int a_fmt, const float* sA, int sa_rows,
                           const void* B, int b_fmt, const float* sB,
                           void* C, const int32_t* group_offsets,
                           int num_groups, int64_t M_total, int64_t N, int64_t K,
                           int out_dtype, hipStream_t stream);

/*
 * dg_grouped_gemm_fp8_ex for padded segments whose real row counts are
 * known: the padding-aware form of the one-launch grouped GEMM (experts'
 * row counts vary, FP8-for-MoE page, section 2.2; padding every segment to
 * the 128-row tile multiplies rows that carry no token).
 *
 *   group_counts : DEVICE int32 [num_groups]; expert e has group_counts[e]
 *                  real rows, rows [o_e, o_e + group_counts[e]) of its
 *                  segment, and 0 <= group_counts[e] <= o_{e+1} - o_e.
 *
 * Rows [o_e + group_counts[e], o_{e+1}) are padding: their rows of C are
 * written as zeros, whatever A and sA hold there (they need not be zeroed
 * by the caller).  Tiles and 64-row wave sub-tiles that lie wholly in
 * padding skip the products (a wave of padding rows still takes part in the
 * workgroup's loads).  Real rows are computed exactly as by
 * dg_grouped_gemm_fp8_ex; with every count equal to its segment length the
 * result is that call's, bit for bit.  Counts outside [0, segment length]
 * are clamped into it (DG_VALIDATE=1 rejects them with DG_ERR_INVALID_ARG);
 * group_counts null or not 4-byte aligned -> DG_ERR_INVALID_ARG.  Everything
 * else as for dg_grouped_gemm_fp8_ex.
 */
int dg_grouped_gemm_fp8_ex_counts(const void* A, int a_fmt, const float* sA, int sa_rows,
                                  const void* B, int b_fmt, const float* sB,
                                  void* C, const int32_t* group_offsets,
                                  const int32_t* group_counts, int num_groups,
                                  int64_t M_total, int64_t N, int64_t K,
                                  int out_dtype, hipStream_t stream);

/*
 * MoE grouped GEMM for few rows per expert (decode), over UNPADDED expert
 * segments, in one launch.  MoE experts share N and K while the row count
 * varies and is small at decode time (FP8-for-MoE page, section 2.2); many
 * small GEMMs, whose launch cost rivals their run time, are better merged
 * into one launch (same page, section 5.2).  Padding every expert's rows to
 * 128 would multiply the work of a decode step many times over, so here the
 * segments are packed: rows [o_e, o_{e+1}) of A and C belong to expert e for
 * ANY 0 = o_0 <= o_1 <= ... <= o_G = M_total.  A scale block of 128 rows
 * would then mix experts, so A carries one scale per row (the 1 x 128
 * granularity of the FP8 kernel write-up, section 5.2):
 *
 *   A             : a_fmt bytes [M_total][K]
 *   sA            : float32 [M_total][Kb]
 *   B             : b_fmt bytes [num_groups][N][K]
 *   sB            : float32 [num_groups][ceil(N/128)][Kb]
 *   C             : [M_total][N] float32 or bfloat16
 *   group_offsets : DEVICE int32 [num_groups + 1] as above
 *
 *   C[i][j] = sum_kb fp32(sA[i][kb] * sB_e[j/128][kb]) * P_kb[i][j] for i in
 *   expert e's segment, P_kb as in dg_gemm_fp8_blockscaled with B_e.
 *
 * Tuned for segments of at most 64 rows: B_e is then streamed from HBM once
 * and an expert without rows costs nothing but reading its two offsets.
 * Longer segments are correct but re-stream B_e once per 64 rows (use
 * dg_grouped_gemm_fp8 for prefill-sized segments).  Offsets are not
 * validated on the host (except under DG_VALIDATE=1, as for
 * dg_grouped_gemm_fp8, here without the multiple-of-128 rule); the kernel
 * clamps them into [0, M_total], so offsets that break the rules give wrong
 * rows but no out-of-bounds access.
 * Host-side errors: num_groups < 1, unknown formats -> DG_ERR_INVALID_ARG;
 * the shared rules above otherwise (M_total need not be a multiple of 128).
 */
int dg_grouped_gemm_fp8_segments(const void* A, int a_fmt, const float* sA,
                                 const void* B, int b_fmt, const float* sB,
                                 void* C, const int32_t* group_offsets,
                                 int num_groups, int64_t M_total, int64_t N, int64_t K,
                                 int out_dtype, hipStream_t stream);

typedef enum {
  DG_IN_F32 = 0,    /* X is float32 */
  DG_IN_BF16 = 1    /* X is bfloat16 */
} dg_in_dtype;

/*
 * FP8 (E4M3FN) block quantisation of activations: the step that produces the
 * A operand and its scales, re-run on every inference (block-wise scaling,
 * FP8-for-MoE page, section 2.1, activations re-scaled at run time, section
 * 4.3; amax-based dynamic scaling, the low-precision essay,
 * hotelren.com/news/5702847, section 2.1).  Per block of block_rows rows x
 * 128 columns:
 *
 *   amax = max |x|;   s = fp32(amax / 448), or 1 if the block is all zero;
 *   Q    = the E4M3FN code nearest to x / s (quotient in double precision),
 *          ties to the even code, magnitude capped at 448, sign bit of x.
 *
 *   X          : [M][K] row-major, in_dtype (DG_IN_F32 or DG_IN_BF16)
 *   Q          : E4M3FN bytes [M][K] row-major (the layout A of the GEMMs takes)
 *   S          : float32 [ceil(M / block_rows)][K/128] row-major
 *   block_rows : 128 (the 128 x 128 blocks the GEMM entry points consume as
 *                sA) or 1 (one scale per token and 128-column group, the
 *                1 x 128 granularity of the FP8 kernel write-up, section 5.2)
 *
 * Shared conventions above apply (caller-owned device memory, asynchronous on
 * `stream`, host-side argument checks).  X and Q must be 16-byte aligned, S
 * 4-byte aligned.  DG_ERR_INVALID_ARG: unknown in_dtype or block_rows,
 * negative or too large sizes, null or misaligned pointers for non-empty
 * work.  DG_ERR_UNSUPPORTED: K not a multiple of 128 or above 2^22.  M == 0 or
 * K == 0 is a no-op.  Non-finite inputs give unspecified codes (never a
 * fault).
 */
int dg_quantize_fp8_blockscaled(const void* X, int in_dtype, void* Q, float* S,
                                int64_t M, int64_t K, int block_rows,
                                hipStream_t stream);

/* Static, NUL-terminated description of a dg_status value. */
const char* dg_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* DG_H_ */
