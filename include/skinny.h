/*
 * skinny.h -- C ABI of the MI355X (gfx950) weight-streaming skinny matmul.
 *
 * The operation is C[m,n] = A[m,k] . W[k,n] for small-to-moderate m, the
 * product the nx_batchscale_kat page asks about ("is the matmul amortising
 * across m?"): W is read from HBM once per call for all m rows.  Around it sit
 * the steps the Strata PR #109 page ("What") batches over a decode window --
 * the router's multi-row GEMV and per-row top-10, the shared expert's scalar
 * gate, the bf16 cast of the window's rows and the MoE combine -- and the f16
 * dequant of a block-quantised weight from the opus r35 track A page
 * (section 1, `dq_f16`), fused into the weight load path.
 *
 * Layouts (all row-major, element strides):
 *   A  [m][lda]   f16 or bf16 rows ("tokens"), or fp32 rows that a bf16-weight
 *                 GEMV rounds to bf16 as it loads them; lda >= k
 *   W  [n][k]     the weight stored k-contiguous: stored row j is logical
 *                 column j of W[k,n].  f16, bf16, Q8_0, Q4_0 or Q2_0 (see below)
 *   C  [m][ldc]   f32, f16 or bf16; ldc >= n
 * Q8_0-style weights are two arrays: codes int8 [n][k] and scales f16
 * [n][k/32]; weight (j, kk) is RNE_f16(scale[j][kk/32] * code[j][kk]).
 * Q4_0-style weights (a 4-bit block format: the Strata PR #109 page,
 * "Measured", names 4- and 2-bit formats without defining one, so this one
 * is fixed here) are codes uint8 [n][k/2] -- two unsigned 4-bit codes q per
 * byte, element kk in byte kk/2, the low nibble for even kk and the high
 * nibble for odd kk -- and scales f16 [n][k/32]; weight (j, kk) is
 * RNE_f16(scale[j][kk/32] * (q - 8)).
 * Q2_0-style weights (the 2-bit format the same page names, Q2_0 runs, also
 * without a definition; fixed here as the 2-bit counterpart of Q4_0) are
 * codes uint8 [n][k/4] -- four unsigned 2-bit codes q per byte, element kk
 * in byte kk/4 at bits 2*(kk%4) and 2*(kk%4)+1 -- and scales f16 [n][k/32];
 * weight (j, kk) is RNE_f16(scale[j][kk/32] * (q - 2)).
 *
 * Paths: m <= 16 runs a multi-row GEMV (every W byte read once for all rows);
 * m >= 17 runs an f16/bf16 MFMA GEMM with a tile chosen by the plan.
 * Guarantees (bitwise):
 *   - row invariance in the GEMV regime: row i of C at any m <= 16 equals the
 *     m = 1 call on that row (Strata PR #109, "What": outputs of the batched
 *     window are bit-identical to the per-token calls);
 *   - tile invariance and M invariance in the GEMM regime: every tile, and
 *     every m >= 17, gives the same bits for the same A row (opus r35 track A,
 *     section 2 and "verification": all tiles memcmp-equal);
 *   - the fused Q8_0 (Q4_0, Q2_0) path equals skinny_dequant_q8_0_run
 *     (skinny_dequant_q4_0_run, skinny_dequant_q2_0_run) followed by the f16
 *     path on the dequantised weight.
 * Across the two regimes results agree to rounding only.
 *
 * Memory and threading:
 *   - every device pointer is owned by the caller; the library keeps none;
 *   - a plan is host memory only, immutable after creation, and may be used
 *     from several threads and streams at once;
 *   - the run calls allocate nothing, never synchronise, and only enqueue
 *     kernels on `stream` (a hipStream_t; NULL = the null stream), so they can
 *     be captured in a HIP graph;
 *   - the optional workspace is caller-owned scratch; two runs in flight at
 *     once must not share one workspace.
 * Errors: every argument is checked on the host before any HIP call; on an
 * error nothing is enqueued and nothing is written.  The library never aborts
 * and prints nothing unless SKINNY_LOG=1 is set.  Non-finite inputs are
 * outside the contract (they propagate as IEEE arithmetic makes them).
 */
#ifndef SKINNY_H
#define SKINNY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SKINNY_ABI_VERSION 1

#if defined(__GNUC__)
#define SKINNY_API __attribute__((visibility("default")))
#else
#define SKINNY_API
#endif

typedef enum skinny_status {
  SKINNY_OK = 0,
  SKINNY_ERR_INVALID_ARG = 1, /* null pointer, bad struct_size, m/n/k/topk out of range */
  SKINNY_ERR_UNSUPPORTED = 2, /* dtype combination or flag the library does not implement */
  SKINNY_ERR_ALIGNMENT = 3,   /* pointer not 16-byte aligned or lda not a multiple of 8 */
  SKINNY_ERR_SHAPE = 4,       /* k not a multiple of 8 (32 for the block formats), stride < row length, a
                                 size past a stated limit (a run: a GEMV of more than about
                                 2^31 waves, k/512 x n) */
  SKINNY_ERR_HIP = 5,         /* the HIP runtime reported an error (device query or launch) */
  SKINNY_ERR_WORKSPACE = 6,   /* workspace missing or smaller than skinny_mm_workspace_size */
  SKINNY_ERR_SCRATCH = 7      /* skinny_mm_run_static: the run needs more scratch than the
                                 library's static array holds (SKINNY_STATIC_*_BYTES) */
} skinny_status;

typedef enum skinny_dtype {
  SKINNY_F16 = 1,
  SKINNY_BF16 = 2,
  SKINNY_F32 = 3,
  SKINNY_Q8_0 = 4,
  SKINNY_Q4_0 = 5,
  SKINNY_Q2_0 = 6
} skinny_dtype;

/* desc.flags */
#define SKINNY_FORCE_GEMV 0x1u /* use the GEMV for every m (m must stay <= 16) */
#define SKINNY_FORCE_GEMM 0x2u /* use the MFMA GEMM for every m, including m <= 16 */
/* A plan whose GEMM cuts k into chunks (narrow n) can run them as one block
 * per chunk plus an ordered reduce launch, or as one launch that folds the
 * chunk sums in the same order; both give the same bits and the plan picks
 * the faster per m.  These flags force one shape (tests); with the second, a
 * tile that cannot hold two accumulator sets falls back to the first. */
#define SKINNY_GEMM_SPLIT_LAUNCH 0x4u
#define SKINNY_GEMM_ONE_LAUNCH 0x8u
/* A third shape, one launch with one block per (tile, chunk) in which the
 * last block of each tile to finish adds the tile's chunk sums in chunk order
 * (the same bits again; no reduce launch, arrival counters in the
 * workspace).  It measured slower than the other two on MI355X, so a plan
 * runs it only when this flag asks for it; tiles that cannot run it use the
 * split launch.  At most one of the three shape flags may be set. */
#define SKINNY_GEMM_FOLD_LAUNCH 0x20u
/* C = sigmoid(A . W) elementwise, sigmoid(x) = 1 / (1 + e^-x) in fp32 (the
 * Strata PR #109 page, "What": the shared expert's scalar gate is a
 * multi-row GEMV followed by a sigmoid; here the sigmoid is applied as the
 * GEMV stores each output, so no second launch runs).  GEMV regime only, for
 * the gate's bf16 weight: the plan needs max_m <= 16, no SKINNY_FORCE_GEMM,
 * w_dtype SKINNY_BF16 and c_dtype SKINNY_F32 or SKINNY_F16 (else
 * SKINNY_ERR_UNSUPPORTED), and gemv_topk_run rejects such a plan.  The
 * sigmoid acts on each output alone, so row invariance holds. */
#define SKINNY_EPILOGUE_SIGMOID 0x10u

#define SKINNY_GEMV_MAX_M 16
#define SKINNY_TOPK_MAX 32

/* Problem description, copied into the plan.
 *   struct_size  sizeof(skinny_mm_desc), for ABI versioning
 *   a_dtype      SKINNY_F16 or SKINNY_BF16; or SKINNY_F32 with bf16 weights in
 *                the GEMV regime (max_m <= 16, no SKINNY_FORCE_GEMM; else
 *                SKINNY_ERR_UNSUPPORTED): fp32 rows whose values the GEMV
 *                rounds to bf16 (nearest even) as it loads them -- the
 *                window-row cast below fused into the GEMV, so C equals the
 *                result for the cast rows bit for bit, in one launch
 *   w_dtype      SKINNY_F16 / SKINNY_Q8_0 / SKINNY_Q4_0 / SKINNY_Q2_0 (with f16 A) or
 *                SKINNY_BF16 (with bf16 or f32 A)
 *   c_dtype      SKINNY_F32, SKINNY_F16 or SKINNY_BF16 (rounded to nearest even)
 *   max_m        largest m any run will pass (>= 1)
 *   n, k         output columns and reduction length (n >= 1; k >= 8, k % 8 == 0,
 *                k % 32 == 0 for Q8_0, Q4_0 and Q2_0; k and lda <= 2^20, k >= 64
 *                for those three
 *                and max_m * n <= 2^50 when the plan may use the GEMM, i.e.
 *                max_m > 16 or SKINNY_FORCE_GEMM)
 *   lda, ldc     row strides of A and C in elements; 0 means dense (k and n);
 *                otherwise >= the row length; lda a multiple of 8 (A rows are
 *                read 16 bytes at a time, 32 for fp32 rows), ldc any value >= n
 *   flags        SKINNY_FORCE_* (tests and benchmarks); 0 normally
 *   tile_id      -1: the plan's tile selector; >= 0: force that GEMM tile
 *                (see skinny_gemm_tile_count)
 *   num_cus      0: query the current HIP device; > 0: plan for that many
 *                compute units without touching the device (host-only use) */
typedef struct skinny_mm_desc {
  uint32_t struct_size;
  int32_t a_dtype;
  int32_t w_dtype;
  int32_t c_dtype;
  int64_t max_m;
  int64_t n;
  int64_t k;
  int64_t lda;
  int64_t ldc;
  uint32_t flags;
  int32_t tile_id;
  int32_t num_cus;
} skinny_mm_desc;

typedef struct skinny_plan skinny_plan;

/* Validate `desc` and build a plan: the GEMV work split (fixed by n and k
 * only, so every m sees the same per-row arithmetic) and the GEMM tile for
 * each m (opus r35 track A, section 2: a tile whose tail block is up to half
 * padding loses, so the selector avoids it).  Host memory only. */
SKINNY_API skinny_status skinny_mm_plan(const skinny_mm_desc* desc, skinny_plan** out_plan);

/* Free a plan (NULL is ignored).  Runs already enqueued are unaffected. */
SKINNY_API void skinny_mm_plan_destroy(skinny_plan* plan);

/* Bytes of device workspace a run with this plan may need (0 when none);
 * enough for every m <= max_m, for skinny_mm_run and gemv_topk_run alike.
 * Three kinds of run need it:
 *   - a GEMV whose k is split into more pieces than one workgroup sums
 *     (k > 8192 for 16-bit weights): it holds the arrival counters (first)
 *     and the fp32 partial sums that let the last wave of each column range
 *     finish the sum inside the same kernel;
 *   - a GEMM whose plan cuts k into chunks (narrow n) and runs them as one
 *     block per chunk: it holds the chunks' fp32 partial sums, which an
 *     ordered reduce launch adds (or, with SKINNY_GEMM_FOLD_LAUNCH, the
 *     arrival counters per tile and the chunk sums the last block adds);
 *   - a plan with fp32 A whose GEMV splits k (k > 1024 for bf16 weights), at
 *     m > 10, unless its one-row launch fills at most half the CUs m times
 *     over (then each row runs as its own workgroup row, fused): the fused
 *     cast measured slower there than a separate cast launch, so the run
 *     casts the rows into the workspace (after any partial sums) and the
 *     bf16 GEMV reads them -- the same bits as the fused launch.
 * It must be zero-filled once before its first use; every completed run
 * leaves it ready for the next (its counters back at zero).  A run that needs
 * no workspace ignores it. */
SKINNY_API skinny_status skinny_mm_workspace_size(const skinny_plan* plan, size_t* bytes);

/* C[0:m, 0:n] = A[0:m, :] . W  (nx_batchscale_kat: the product with fp32
 * accumulation; Strata PR #109 "What": every W byte read once for the window).
 *   m          1 <= m <= max_m
 *   A, W, C    device pointers (16-byte aligned); w_scales: Q8_0 / Q4_0 / Q2_0 scales
 *              f16 [n][k/32] (16-byte aligned), else must be NULL
 *   workspace  zero-initialised device scratch of >= skinny_mm_workspace_size
 *              bytes (may be NULL when that size is 0)
 *   stream     hipStream_t (NULL = null stream)
 * Enqueues one launch (the GEMV, whose k splits are summed inside it, or the
 * GEMM), or two when the plan's GEMM runs its k chunks as separate blocks
 * (the second adds the chunks in order) or its fp32 rows are cast first (see
 * skinny_mm_workspace_size).  Writes rows 0..m-1 of C, columns
 * 0..n-1 only. */
SKINNY_API skinny_status skinny_mm_run(const skinny_plan* plan, int64_t m, const void* A, const void* W,
                            const void* w_scales, void* C, void* workspace,
                            size_t workspace_bytes, void* stream);

/* skinny_mm_run without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It computes what skinny_mm_run computes,
 * with the same kernels, bit for bit, but a run that needs scratch (the
 * cases listed under skinny_mm_workspace_size) uses the library's own static
 * device array instead of a caller's workspace.  It allocates nothing and
 * calls no allocating routine.
 *   The array is SKINNY_STATIC_SCRATCH_BYTES per GPU, held by every GPU the
 *   library runs on until the process ends: SKINNY_STATIC_COUNTER_BYTES of
 *   arrival counters, the rest for partial sums and cast rows.  A run that
 *   needs more (its skinny_mm_workspace_size counters beyond the first
 *   region, or its partial sums and cast rows beyond the second) returns
 *   SKINNY_ERR_SCRATCH before any HIP call; so does nothing else.
 *   The current device's copy is used: `stream` must belong to the current
 *   device (else SKINNY_ERR_HIP).  The first call on a device looks up the
 *   array's device address and enqueues a zero fill of its counter region on
 *   `stream` before the run; every run leaves the counters at zero again.
 *   Every call on one GPU shares that GPU's array, which keeps the last
 *   call's contents: two calls in flight at once on one GPU (on different
 *   streams, or from different threads without ordering) race and may give
 *   wrong results; calls ordered on one stream do not.
 * Other arguments, ownership and errors as skinny_mm_run. */
#define SKINNY_STATIC_SCRATCH_BYTES (32u << 20)
#define SKINNY_STATIC_COUNTER_BYTES (1u << 20)
SKINNY_API skinny_status skinny_mm_run_static(const skinny_plan* plan, int64_t m, const void* A,
                                              const void* W, const void* w_scales, void* C, void* stream);

/* Router step (Strata PR #109, "What": one multi-row router GEMV launch into
 * fp32 logits, then one multi-row top-k launch with a wavefront per row).
 * The workspace is as for skinny_mm_run.  The plan's c_dtype must be
 * SKINNY_F32.
 *   logits     f32 [m][ldc] out (the full product)
 *   topk_idx   int32 [m][topk] out: the topk largest logits of each row,
 *              value descending, equal values (IEEE ==, so -0 == +0) by lower
 *              column index first
 *   topk_val   f32 [m][topk] out: those logits, bit-for-bit
 *   topk       1 <= topk <= min(n, SKINNY_TOPK_MAX) */
SKINNY_API skinny_status gemv_topk_run(const skinny_plan* plan, int64_t m, const void* A, const void* W,
                            const void* w_scales, float* logits, int32_t* topk_idx,
                            float* topk_val, int32_t topk, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Standalone Q2_0-style dequant, the 2-bit format above:
 * out[j][kk] = RNE_f16(f32(d[j][kk/32]) * (q - 2)), q the 2-bit code of
 * element kk (bits 2*(kk%4) and 2*(kk%4)+1 of qs[j][kk/4]); the same
 * arithmetic the fused paths use.
 *   n >= 1, k >= 32 and k % 32 == 0; qs uint8 [n][k/4], d f16 [n][k/32],
 *   out f16 [n][k]; all device pointers, 16-byte aligned. */
SKINNY_API skinny_status skinny_dequant_q2_0_run(int64_t n, int64_t k, const void* qs, const void* d,
                                      void* out, void* stream);

/* Standalone Q4_0-style dequant, the 4-bit format above:
 * out[j][kk] = RNE_f16(f32(d[j][kk/32]) * (q - 8)), q the 4-bit code of
 * element kk (low nibble of qs[j][kk/2] for even kk, high nibble for odd);
 * the same arithmetic the fused paths use.
 *   n >= 1, k >= 32 and k % 32 == 0; qs uint8 [n][k/2], d f16 [n][k/32],
 *   out f16 [n][k]; all device pointers, 16-byte aligned. */
SKINNY_API skinny_status skinny_dequant_q4_0_run(int64_t n, int64_t k, const void* qs, const void* d,
                                      void* out, void* stream);

/* Standalone Q8_0-style dequant (opus r35 track A, section 1: `dq_f16`):
 * out[j][kk] = RNE_f16(f32(d[j][kk/32]) * f32(qs[j][kk])), the same
 * arithmetic the fused paths use.
 *   n >= 1, k >= 32 and k % 32 == 0; qs int8 [n][k], d f16 [n][k/32],
 *   out f16 [n][k]; all device pointers, 16-byte aligned. */
SKINNY_API skinny_status skinny_dequant_q8_0_run(int64_t n, int64_t k, const void* qs, const void* d,
                                      void* out, void* stream);

/* The window-row cast (the Strata PR #109 page, "What": the window's fp32
 * rows are cast to bf16 in one call, the rows being contiguous):
 * out[i] = RNE_bf16(in[i]) for 0 <= i < count, round to nearest, ties to
 * even; a NaN becomes a quiet NaN.  The result feeds a bf16 plan's A (a plan
 * with fp32 A does the same rounding inside its one GEMV launch).
 *   1 <= count <= 2^40; in: f32 [count], out: bf16 [count]; device pointers,
 *   16-byte aligned, not overlapping (else SKINNY_ERR_INVALID_ARG). */
SKINNY_API skinny_status skinny_cast_f32_bf16_run(int64_t count, const float* in, void* out, void* stream);

/* The MoE combine (the Strata PR #109 page, "What": one combine launch for
 * the window's tokens, the token taken from the grid's y index):
 *   out[t][c] = sum over i < topk of weights[t][i] * rows[t][i][c]
 *               + gate[t] * shared_rows[t][c]     (when shared_rows is given)
 * accumulated in fp32, experts in order i = 0 .. topk - 1 and the shared
 * term last, each as one fused multiply-add, then rounded once to out_dtype
 * (nearest even for bf16).  The page does not say how the routing weights
 * are formed; the caller passes them.  Each token's row is computed on its
 * own, so it does not depend on m.
 *   m >= 1 tokens; d >= 8 with d % 8 == 0 (else SKINNY_ERR_SHAPE);
 *   1 <= topk <= SKINNY_TOPK_MAX; m * topk * d <= 2^56
 *   rows         [m][topk][d] expert output rows, SKINNY_F32 or SKINNY_BF16
 *                (rows_dtype); 16-byte aligned
 *   weights      f32 [m][topk] routing weights; 4-byte aligned
 *   shared_rows  [m][d] in rows_dtype (16-byte aligned) and gate f32 [m]
 *                (4-byte aligned): both or neither (else SKINNY_ERR_INVALID_ARG)
 *   out          [m][d] SKINNY_F32 or SKINNY_BF16 (out_dtype), 16-byte aligned,
 *                overlapping no input (else SKINNY_ERR_INVALID_ARG)
 * All device pointers.  One launch. */
SKINNY_API skinny_status skinny_moe_combine_run(int64_t m, int64_t d, int32_t topk, const void* rows,
                                     const float* weights, const void* shared_rows, const float* gate,
                                     int32_t rows_dtype, void* out, int32_t out_dtype, void* stream);

/* Human-readable description of what a run with this m would launch: path,
 * tile or GEMV split, grid.  Writes a NUL-terminated string (truncated to
 * len). */
SKINNY_API skinny_status skinny_mm_plan_info(const skinny_plan* plan, int64_t m, char* buf, size_t len);

/* Number of GEMM tiles and the name of tile `tile_id` ("TMxTN_wWMxWN"). */
SKINNY_API int32_t skinny_gemm_tile_count(void);
SKINNY_API const char* skinny_gemm_tile_name(int32_t tile_id);

/* Static text for a status code. */
SKINNY_API const char* skinny_status_string(skinny_status status);

/* SKINNY_ABI_VERSION of the built library. */
SKINNY_API int32_t skinny_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SKINNY_H */
