// internal.h -- host-side interfaces between the C ABI (abi.cpp) and the
// kernel translation units (gemv.hip, gemm.hip).  Not installed.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace skinny {

// weight storage kinds and output kinds (kernel template parameters)
enum WKind : int { WK_F16 = 0, WK_BF16 = 1, WK_Q8 = 2, WK_Q4 = 3, WK_Q2 = 4 };
enum CKind : int { CK_F32 = 0, CK_F16 = 1, CK_BF16 = 2 };

// ---------------------------------------------------------------------------
// Multi-row GEMV (m <= 16).  One wavefront owns a k-range of 64*T chunks of
// eight elements (chunk c = split*64*T + t*64 + lane) and a run of `cpw`
// consecutive columns; its A slice lives in registers for the whole wave.
// The k split (T, S) depends on k only, so the per-row arithmetic is the same
// for every m.
// ---------------------------------------------------------------------------
constexpr int kGemvMaxM = 16;
constexpr int kGemvCpwMax = 8;     // columns per wave, upper bound
constexpr int kGemvMaxWavesPerBlock = 8;
// k splits up to this many are summed inside one workgroup (through LDS);
// beyond it through fp32 partials in the caller's workspace
constexpr int kGemvBlockSplitMax = 8;

struct GemvArgs {
  const void* A;           // [m][lda] f16/bf16 bits, or fp32 (a_kind = kAF32)
  int64_t lda;
  const void* W;           // [n][k] f16/bf16 bits, int8 codes (Q8_0), or packed 4-bit codes
                           // [n][k/2] (Q4_0) or 2-bit codes [n][k/4] (Q2_0)
  const uint16_t* scales;  // block formats: scales [n][k/32] (f16 bits), else null
  int64_t n;
  int64_t k;
  int32_t nchunks;          // k / 8
  int32_t S;                // number of k splits
  int32_t cpw;              // columns per wave (1..kGemvCpwMax)
  int32_t waves_per_split;  // ceil(n / cpw)
  int32_t cg_per_block;     // S <= kGemvBlockSplitMax: column ranges per block (S waves each)
  void* C;                  // [m][ldc] output
  int64_t ldc;
  float* partial;           // [S][m][n] fp32 partial sums (S > kGemvBlockSplitMax)
  uint32_t* counters;       // [waves_per_split] arrivals per column range (S > kGemvBlockSplitMax),
                            // zero between calls
  int32_t epilogue;         // kEpiNone, or kEpiSigmoid: C = 1 / (1 + e^-sum)
  int32_t a_kind;           // kA16, or kAF32 (bf16 weights only)
  uint32_t wave_range;      // S <= kGemvBlockSplitMax: 4 bits per wave w of a workgroup, w / S
  uint32_t wave_split;      //   and w % S (no division in the kernel)
  int32_t row_groups;       // workgroup rows of the grid: row y of the grid takes rows y*m ..
                            // y*m + m - 1 of A and C (more than one only for S <= 8)
};

constexpr int kEpiNone = 0;
constexpr int kEpiSigmoid = 1;

// A rows: kA16 -- the weights' own 16-bit type; kAF32 -- fp32, each value
// rounded to bf16 (nearest even) as it is loaded
constexpr int kA16 = 0;
constexpr int kAF32 = 1;

// out_kind: 0 f32, 1 f16, 2 bf16 (C)
hipError_t launch_gemv(const GemvArgs& args, int m, int T, int w_kind, int out_kind,
                       int waves_per_block, hipStream_t stream);

// Per-row top-k of f32 rows written by an earlier launch, one wavefront per
// row (blockIdx.x = row).
hipError_t launch_topk(const float* logits, int m, int64_t n, int64_t ldl, int32_t* idx, float* val,
                       int topk, hipStream_t stream);

// out[i] = bf16(in[i]) (round to nearest even) for i < count
hipError_t launch_cast_f32_bf16(int64_t count, const float* in, uint16_t* out, hipStream_t stream);

hipError_t launch_dequant_q8_0(int64_t n, int64_t k, const int8_t* qs, const uint16_t* d,
                               uint16_t* out, hipStream_t stream);
hipError_t launch_dequant_q4_0(int64_t n, int64_t k, const uint8_t* qs, const uint16_t* d,
                               uint16_t* out, hipStream_t stream);
hipError_t launch_dequant_q2_0(int64_t n, int64_t k, const uint8_t* qs, const uint16_t* d,
                               uint16_t* out, hipStream_t stream);

// MoE combine: out[t][c] = sum_i w[t][i] * rows[t][i][c] (+ gate[t] * shared[t][c])
struct CombineArgs {
  int64_t m;             // tokens
  int64_t d;             // row length (d % 8 == 0)
  int64_t topk;          // expert rows per token
  const void* rows;      // [m][topk][d] fp32 or bf16
  const float* weights;  // [m][topk]
  const void* shared;    // [m][d] like rows, or null (then gate is not read)
  const float* gate;     // [m]
  void* out;             // [m][d] fp32 or bf16
};

constexpr int kCombineMaxTopk = 32;  // expert rows per token the combine takes

// rows_kind / out_kind: CK_F32 or CK_BF16
hipError_t launch_moe_combine(const CombineArgs& args, int rows_kind, int out_kind, hipStream_t stream);

// ---------------------------------------------------------------------------
// MFMA GEMM (v_mfma_f32_32x32x16_{f16,bf16} for every tile, K-tiles of 32 in
// increasing k, so every tile gives the same bits).
// ---------------------------------------------------------------------------
// largest k (and lda) the GEMM path takes: a block's rows of A and W are
// addressed with 32-bit byte offsets
constexpr int64_t kGemmMaxK = 1 << 20;

struct GemmArgs {
  const uint16_t* A;       // [M][lda]
  int64_t lda;
  const void* W;           // [N][K] (f16/bf16 bits, int8 codes, or packed 4-bit codes [N][K/2]
                           // or 2-bit codes [N][K/4])
  const uint16_t* scales;  // block formats: scales [N][K/32]
  int64_t M;
  int64_t N;
  int64_t K;
  void* C;                 // [M][ldc]
  int64_t ldc;
  int32_t splits;          // blocks per tile: k split into this many ranges of
  int32_t kt_per_split;    // kt_per_split k-tiles (also the chunk of a chunked launch)
  float* partial;          // splits > 1: [splits][M][N] fp32 partial sums (split launch), or
                           // [tile][split][TM * TN] chunk sums in register order (fold launch)
  uint32_t* counters;      // fold launch: arrivals per tile, zero between calls
};

struct GemmTileInfo {
  int tm, tn, wm, wn;  // block tile and wave grid (each wave owns (tm/wm) x (tn/wn))
  const char* name;
};

int gemm_tile_count();
const GemmTileInfo& gemm_tile(int id);

// Launch shapes of a plan whose k is cut into chunks (args.splits > 1 for the
// split and fold shapes; 1 for the chunked shape, which walks all chunks):
//   kGemmPlain    one block per tile over all of k (unchunked plans), or one
//                 block per (tile, chunk) writing partial sums for the
//                 reduce launch (splits > 1);
//   kGemmChunked  one block per tile folding its chunk sums in order
//                 (needs a chunkable tile);
//   kGemmFold     one block per (tile, chunk); the last block of a tile to
//                 finish folds the tile's chunk sums in order and writes C.
constexpr int kGemmPlain = 0;
constexpr int kGemmChunked = 1;
constexpr int kGemmFold = 2;
hipError_t launch_gemm(int tile_id, const GemmArgs& args, int w_kind, int c_kind, int shape,
                       hipStream_t stream);
bool gemm_tile_chunkable(int tile_id);
bool gemm_tile_foldable(int tile_id);

// C = sum over s = 0..splits-1, in that order, of partial[s] (fp32), rounded
// to the output kind
hipError_t launch_splitk_reduce(const GemmArgs& args, int c_kind, hipStream_t stream);

// ---------------------------------------------------------------------------
// The library's own scratch for skinny_mm_run_static: one file-scope device
// array per GPU (static_scratch.hip), [counters: kStaticCounterBytes]
// [data: the rest].  static_scratch() returns the current device's address of
// it; on its first call on a device it looks the address up and enqueues a
// zero fill of the counter region on `stream`.
// ---------------------------------------------------------------------------
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr size_t kStaticCounterBytes = size_t(1) << 20;
constexpr size_t kStaticDataBytes = kStaticScratchBytes - kStaticCounterBytes;

hipError_t static_scratch(hipStream_t stream, char** base);

}  // namespace skinny
