// gemm.hip -- f16 / bf16 MFMA GEMM for the m >= 17 regime on gfx950 (MI355X).
//
// C[M,N] = A[M,K] . W[K,N] with W stored [N][K] (both operands k-contiguous),
// fp32 accumulation in the matrix cores, f32/f16/bf16 output.
//
// What the pages fix, and how it is met here:
//   * opus r35 track A, section 2 ("gemm_f16 tiles"): a family of tiles
//     TM x TN whose results are bitwise identical, chosen per M.  Here every
//     tile issues the same instruction, v_mfma_f32_32x32x16_{f16,bf16}, with
//     the same operand layout, and accumulates every output in one register
//     over k = 0, 16, 32, ... in increasing order, and every tile origin is a
//     multiple of 32 rows and columns.  So an output element sees the same
//     arithmetic under every tile and every M (tile- and M-invariance).
//   * the same section's tail rule (a 128-row tile whose last block is up to
//     half padding loses): rows past M are zero-filled in LDS and masked on
//     store; the plan's selector counts padded tiles when it picks a tile.
//   * opus r35 track A, section 1 (`dq_f16` before the router GEMM): the Q8_0
//     B-loader dequantises each k-tile of a weight row straight into the f16
//     LDS tile with the same function as the standalone dequant, so no
//     separate dequant pass or f16 copy of the weight exists.
//   * Strata PR #109 ("Measured"): results must not depend on a split of the
//     reduction; there is no split-k.
//
// Structure (64-wide wavefronts, 4 waves in a 2 x 2 grid for the main tiles):
//   * k-tiles of 64 (four MFMA steps per barrier);
//   * global loads run two k-tiles ahead (16-byte, coalesced: 8 lanes cover
//     one 128-byte row segment) into two register sets; a tile's registers
//     are written to the other LDS buffer half way through the MFMAs of the
//     tile before it, so a k-tile and a half of MFMA work hides their latency
//     (256 x 256 tiles, whose accumulators fill the register file, keep one
//     set: loaded at the start of a tile, written after its MFMAs);
//   * blocks are renumbered so that each XCD (blocks b, b + 8, ... share one)
//     runs a contiguous range of tiles in column-major order: the weight
//     columns an XCD needs stay in its own L2 instead of all eight;
//   * LDS rows are 128 bytes (eight 16-byte chunks); chunk c of row r is
//     stored at c ^ ((r >> 1) & 7), so the sixteen rows read by sixteen
//     consecutive lanes at one logical chunk hit sixteen different 16-byte
//     bank groups (conflict-free for 64 banks; the bank-conflict counter
//     measured the plain r & 7 swizzle at one stall per two accesses);
//   * MFMA operand fragments are read for step ks + 1 while step ks's MFMAs
//     run; the accumulators of a 128 x 128 wave tile (256 fp32 per lane) live
//     in the accumulation registers.
#include "device_common.h"
#include "internal.h"

namespace skinny {

namespace {

// buffer resource word 3 for raw (unstrided) 32-bit buffers on gfx9-family
// parts; out-of-range offsets read as zero
constexpr int kBufferFlags = 0x00020000;

constexpr int kBK = 64;        // k per LDS tile: four 32x32x16 MFMA steps
constexpr int kCPR = kBK / 8;  // 16-byte chunks per tile row (8)
constexpr int kSteps = kBK / 16;

// LDS rows are 128 bytes; gfx950 serves 16 lanes of a ds_read_b128 per cycle
// from 64 banks (256 bytes), i.e. two rows.  Chunk c of row r goes to
// c ^ ((r >> 1) & 7): the 16 rows read by 16 consecutive lanes at one logical
// chunk then cover all 16 bank groups of the two-row window.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

__device__ __forceinline__ h8_t as_h8(u32x4 v) { return __builtin_bit_cast(h8_t, v); }
__device__ __forceinline__ b8_t as_b8(u32x4 v) { return __builtin_bit_cast(b8_t, v); }

template <int WK>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (WK == WK_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_b8(a), as_b8(b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_h8(a), as_h8(b), c, 0, 0, 0);
  }
}

template <int TM, int TN, int WM, int WN, int WK, int CK>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(GemmArgs g) {
  constexpr int NT = 64 * WM * WN;
  constexpr int WTM = TM / WM;
  constexpr int WTN = TN / WN;
  constexpr int FM = WTM / 32;
  constexpr int FN = WTN / 32;
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
  constexpr int A_CHUNKS = TM * kCPR;
  constexpr int A_ITERS = (A_CHUNKS + NT - 1) / NT;
  // Q8_0 rows arrive as 16-code quarters of a 64-wide k-tile; f16/bf16 rows as 8 chunks
  constexpr int B_UNITS = (WK == WK_Q8) ? TN * 4 : TN * kCPR;
  constexpr int B_ITERS = (B_UNITS + NT - 1) / NT;
  static_assert(A_CHUNKS % NT == 0 && (WK == WK_Q8 || B_UNITS % NT == 0),
                "tile rows must split evenly over the block");
  // register sets for staged k-tiles: two (prefetch distance 2) when the
  // accumulators, both sets, the double-buffered fragments and some slack fit
  // the per-wave register budget (512 registers per SIMD lane shared by the
  // waves of one block on each SIMD), else one (distance 1)
  constexpr int kRegBudget = 512 / ((NT + 255) / 256);
  constexpr int kStageRegs = (A_ITERS + B_ITERS) * 4 + (WK == WK_Q8 ? B_ITERS : 0);
  constexpr int kNeed2 = FM * FN * 16 + 2 * kStageRegs + 2 * (FM + FN) * 4 + 40;
  constexpr int NSETS = kNeed2 <= kRegBudget ? 2 : 1;

  __shared__ u32x4 sA[2][A_CHUNKS];
  __shared__ u32x4 sB[2][TN * kCPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN;
  const int wn = wid - wm * WN;

  // XCD-aware renumbering: hardware block b runs on XCD b % 8; give XCD x the
  // tiles [x * per, (x + 1) * per) of a column-major tile order (the last
  // XCDs may get one fewer), so neighbouring tiles on an XCD share W columns
  const int64_t tiles_m = (g.M + TM - 1) / TM;
  const int64_t nblocks = (int64_t)gridDim.x;
  const int64_t per = (nblocks + 7) / 8;
  const int64_t xcd = blockIdx.x & 7;
  const int64_t full = nblocks - 8 * (per - 1);  // XCDs that get `per` tiles
  const int64_t local = blockIdx.x >> 3;
  const int64_t t = xcd < full ? xcd * per + local : full * per + (xcd - full) * (per - 1) + local;
  const int64_t bn = t / tiles_m;
  const int64_t bm = t - bn * tiles_m;
  const int64_t row0 = bm * TM;
  const int64_t col0 = bn * TN;

  const uint16_t* __restrict__ A = g.A;
  const int64_t K = g.K;  // <= 2^20 (checked by the plan), so offsets fit in 32 bits
  const int nk = (int)((K + kBK - 1) / kBK);

  u32x4 ra[NSETS][A_ITERS];
  u32x4 rb[NSETS][B_ITERS];
  uint16_t rs[NSETS][B_ITERS];  // Q8_0 scale of each staged quarter-row

  // Loads go through buffer resources covering exactly this block's rows of
  // A and W: a row past M or N lies outside the resource and reads as zero
  // (hardware range check), so no load is predicated and the number of loads
  // in flight is the same on every path -- the compiler's vmcnt waits then
  // count exactly.  Each thread keeps one 32-bit offset per operand; the
  // per-iteration row stride and the k-tile origin are scalar offsets.
  // Chunks past K (only when K % 64 != 0) are zeroed by a select when they
  // are written to LDS (a select right after the load would make the wave
  // wait for that load at once).
  const int64_t rows_a = (g.M - row0) < TM ? (g.M - row0) : TM;
  const int64_t rows_b = (g.N - col0) < TN ? (g.N - col0) : TN;
  const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(A + row0 * g.lda), (short)0, (int)(((rows_a - 1) * g.lda + K) * 2), kBufferFlags);
  const int a_r = tid / kCPR;
  const int a_c = tid - a_r * kCPR;
  const int voff_a = (int)((a_r * g.lda + a_c * 8) * 2);
  const bool k_tail = (K % kBK) != 0;

  __amdgpu_buffer_rsrc_t rsrc_b;
  __amdgpu_buffer_rsrc_t rsrc_s;
  int voff_b, voff_s = 0, b_c;
  if constexpr (WK == WK_Q8) {
    rsrc_b = __builtin_amdgcn_make_buffer_rsrc((void*)((const int8_t*)g.W + col0 * K), (short)0,
                                               (int)(rows_b * K), kBufferFlags);
    rsrc_s = __builtin_amdgcn_make_buffer_rsrc((void*)(g.scales + col0 * (K >> 5)), (short)0,
                                               (int)(rows_b * (K >> 5) * 2), kBufferFlags);
    const int b_r = tid >> 2;
    b_c = tid & 3;  // which 16-code quarter of the 64-wide k-tile
    voff_b = (int)(b_r * K + b_c * 16);
    voff_s = (int)((b_r * (K >> 5) + (b_c >> 1)) * 2);
  } else {
    rsrc_b = __builtin_amdgcn_make_buffer_rsrc((void*)((const uint16_t*)g.W + col0 * K), (short)0,
                                               (int)(rows_b * K * 2), kBufferFlags);
    rsrc_s = rsrc_b;
    const int b_r = tid / kCPR;
    b_c = tid - b_r * kCPR;
    voff_b = (int)((b_r * K + b_c * 8) * 2);
  }

  auto load_tiles = [&](int kt, int set) {
    const int k0 = kt * kBK;
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      const int soff = (int)(((int64_t)i * (NT / kCPR) * g.lda + k0) * 2);
      ra[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_a, voff_a, soff, 0));
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      if constexpr (WK == WK_Q8) {
        const int soff = (int)((int64_t)i * (NT / 4) * K + k0);
        const int soff_s = (int)(((int64_t)i * (NT / 4) * (K >> 5) + (k0 >> 5)) * 2);
        rb[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, voff_b, soff, 0));
        rs[set][i] = __builtin_amdgcn_raw_buffer_load_b16(rsrc_s, voff_s, soff_s, 0);
      } else {
        const int soff = (int)(((int64_t)i * (NT / kCPR) * K + k0) * 2);
        rb[set][i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc_b, voff_b, soff, 0));
      }
    }
  };

  auto store_tiles = [&](int buf, int set, int kt) {
    const int k0 = kt * kBK;
    const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      const int r = a_r + i * (NT / kCPR);
      const bool keep = !k_tail || k0 + a_c * 8 < K;
      sA[buf][r * kCPR + (a_c ^ swz(r))] = keep ? ra[set][i] : zero;
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      if constexpr (WK == WK_Q8) {
        const int r = (tid >> 2) + i * (NT / 4);
        // a last, partial pass (TN * 4 not a multiple of the block) loaded
        // rows past the tile, which read as zero; they are not stored
        if (B_UNITS % NT != 0 && r >= TN) continue;
        const bool keep = !k_tail || k0 + b_c * 16 < K;
        const _Float16 d = half_from_bits(keep ? rs[set][i] : (uint16_t)0);
        const u32x4 codes = keep ? rb[set][i] : zero;
        const u32x2 lo = {(uint32_t)codes[0], (uint32_t)codes[1]};
        const u32x2 hi = {(uint32_t)codes[2], (uint32_t)codes[3]};
        sB[buf][r * kCPR + ((2 * b_c) ^ swz(r))] = q8_dequant8(lo, d);
        sB[buf][r * kCPR + ((2 * b_c + 1) ^ swz(r))] = q8_dequant8(hi, d);
      } else {
        const int r = (tid / kCPR) + i * (NT / kCPR);
        const bool keep = !k_tail || k0 + b_c * 8 < K;
        sB[buf][r * kCPR + (b_c ^ swz(r))] = keep ? rb[set][i] : zero;
      }
    }
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int lrow = lane & 31;
  const int lk = lane >> 5;  // which 8-wide half of an MFMA k-step this lane feeds

  // LDS word index of this lane's fragment rows (the chunk is added per step)
  int a_row[FM];
  int b_row[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) a_row[i] = wm * WTM + i * 32 + lrow;
#pragma unroll
  for (int j = 0; j < FN; ++j) b_row[j] = wn * WTN + j * 32 + lrow;

  auto read_frags = [&](int buf, int ks, u32x4 (&af)[FM], u32x4 (&bf)[FN]) {
    const int c = ks * 2 + lk;
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = sA[buf][a_row[i] * kCPR + (c ^ swz(a_row[i]))];
#pragma unroll
    for (int j = 0; j < FN; ++j) bf[j] = sB[buf][b_row[j] * kCPR + (c ^ swz(b_row[j]))];
  };

  // pipeline: tile kt is in LDS buffer kt & 1 when its MFMAs run.  With two
  // register sets, tile kt + 1 sits in set (kt + 1) & 1 and is written to the
  // other buffer half way through tile kt, while tile kt + 2 is loaded into
  // set kt & 1 (emptied during tile kt - 1) at the start of tile kt.  With one
  // set, tile kt + 1 is loaded at the start of tile kt and written after its
  // last MFMA step.
  load_tiles(0, 0);
  if constexpr (NSETS == 2) load_tiles(nk > 1 ? 1 : 0, 1);
  store_tiles(0, 0, 0);
  __syncthreads();

  constexpr int kStoreAfter = (NSETS == 2) ? kSteps / 2 - 1 : kSteps - 1;

  auto tile_step = [&](int kt, int set_next) {
    const int cur = kt & 1;
    // the prefetch is issued on every tile (past the end it re-reads the last
    // tile) and the store on every tile (past the end into a buffer nobody
    // reads), so a tile is one straight-line block with a fixed count of
    // loads in flight
    if constexpr (NSETS == 2) {
      load_tiles(kt + 2 < nk ? kt + 2 : nk - 1, set_next ^ 1);
    } else {
      load_tiles(kt + 1 < nk ? kt + 1 : nk - 1, 0);
    }
    // fragments of step ks + 1 are read while step ks's MFMAs run
    u32x4 af[2][FM];
    u32x4 bf[2][FN];
    read_frags(cur, 0, af[0], bf[0]);
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      if (ks + 1 < kSteps) read_frags(cur, ks + 1, af[(ks + 1) & 1], bf[(ks + 1) & 1]);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<WK>(af[ks & 1][i], bf[ks & 1][j], acc[i][j]);
      if (ks == kStoreAfter) store_tiles(cur ^ 1, NSETS == 2 ? set_next : 0, kt + 1);
    }
    __syncthreads();
  };

  // unrolled by two so the register sets are named at compile time
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    tile_step(kt, 1);
    tile_step(kt + 1, 0);
  }
  if (kt < nk) tile_step(kt, 1);

  // 32x32 accumulator layout: lane owns column (lane & 31); register v holds
  // row 8 * (v / 4) + 4 * (lane / 32) + (v % 4)
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = col0 + wn * WTN + j * 32 + lrow;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = row0 + wm * WTM + i * 32 + 8 * (v >> 2) + 4 * lk + (v & 3);
        if (row < g.M && col < g.N) store_out<CK>(g.C, row * g.ldc + col, acc[i][j][v]);
      }
    }
  }
}

typedef void (*gemm_fn)(GemmArgs);

struct TileEntry {
  GemmTileInfo info;
  gemm_fn fn[3][3];  // [w_kind][c_kind]
};

template <int TM, int TN, int WM, int WN>
TileEntry make_tile(const char* name) {
  TileEntry e;
  e.info = GemmTileInfo{TM, TN, WM, WN, name};
  e.fn[WK_F16][CK_F32] = gemm_kernel<TM, TN, WM, WN, WK_F16, CK_F32>;
  e.fn[WK_F16][CK_F16] = gemm_kernel<TM, TN, WM, WN, WK_F16, CK_F16>;
  e.fn[WK_F16][CK_BF16] = gemm_kernel<TM, TN, WM, WN, WK_F16, CK_BF16>;
  e.fn[WK_BF16][CK_F32] = gemm_kernel<TM, TN, WM, WN, WK_BF16, CK_F32>;
  e.fn[WK_BF16][CK_F16] = gemm_kernel<TM, TN, WM, WN, WK_BF16, CK_F16>;
  e.fn[WK_BF16][CK_BF16] = gemm_kernel<TM, TN, WM, WN, WK_BF16, CK_BF16>;
  e.fn[WK_Q8][CK_F32] = gemm_kernel<TM, TN, WM, WN, WK_Q8, CK_F32>;
  e.fn[WK_Q8][CK_F16] = gemm_kernel<TM, TN, WM, WN, WK_Q8, CK_F16>;
  e.fn[WK_Q8][CK_BF16] = gemm_kernel<TM, TN, WM, WN, WK_Q8, CK_BF16>;
  return e;
}

const TileEntry* tiles() {
  static const TileEntry table[] = {
      make_tile<256, 256, 2, 2>("256x256_w2x2"),
      make_tile<256, 256, 2, 4>("256x256_w2x4"),
      make_tile<256, 128, 4, 2>("256x128_w4x2"),
      make_tile<256, 128, 2, 2>("256x128_w2x2"),
      make_tile<128, 256, 2, 2>("128x256_w2x2"),
      make_tile<128, 128, 2, 2>("128x128_w2x2"),
      make_tile<128, 64, 2, 2>("128x64_w2x2"),
      make_tile<64, 128, 2, 2>("64x128_w2x2"),
      make_tile<64, 64, 2, 2>("64x64_w2x2"),
      make_tile<128, 96, 4, 1>("128x96_w4x1"),
      make_tile<64, 96, 2, 1>("64x96_w2x1"),
      make_tile<32, 96, 1, 1>("32x96_w1x1"),
      make_tile<32, 64, 1, 2>("32x64_w1x2"),
  };
  return table;
}

constexpr int kTileCount = 13;

}  // namespace

int gemm_tile_count() { return kTileCount; }

const GemmTileInfo& gemm_tile(int id) { return tiles()[id].info; }

hipError_t launch_gemm(int tile_id, const GemmArgs& args, int w_kind, int c_kind,
                       hipStream_t stream) {
  if (tile_id < 0 || tile_id >= kTileCount || w_kind < 0 || w_kind > 2 || c_kind < 0 || c_kind > 2)
    return hipErrorInvalidValue;
  const TileEntry& e = tiles()[tile_id];
  const int64_t blocks = ((args.M + e.info.tm - 1) / e.info.tm) * ((args.N + e.info.tn - 1) / e.info.tn);
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(e.fn[w_kind][c_kind], dim3((unsigned)blocks), dim3(64 * e.info.wm * e.info.wn), 0,
                     stream, args);
  return hipGetLastError();
}

}  // namespace skinny
