// gemm.hip -- f16 / bf16 MFMA GEMM for the m >= 17 regime on gfx950 (MI355X).
//
// C[M,N] = A[M,K] . W[K,N] with W stored [N][K] (both operands k-contiguous),
// fp32 accumulation in the matrix cores, f32/f16/bf16 output.
//
// What the pages fix, and how it is met here:
//   * opus r35 track A, section 2 ("gemm_f16 tiles"): a family of tiles
//     TM x TN whose results are bitwise identical, chosen per M.  Here every
//     tile issues the same instruction, v_mfma_f32_32x32x16_{f16,bf16}, with
//     the same k traversal (LDS k-tiles of 32 = two MFMA steps, in increasing
//     k, into one accumulator per output), and every tile origin is a multiple
//     of 32 rows and columns, so an output element sees the same arithmetic
//     under every tile and every M (tile- and M-invariance).
//   * the same section's tail rule (a 128-row tile whose last block is up to
//     half padding loses): rows past M are zero-filled in LDS and masked on
//     store; the plan's selector counts padded tiles when it picks a tile.
//   * opus r35 track A, section 1 (`dq_f16` before the router GEMM): the Q8_0
//     B-loader dequantises each 32-wide k-tile of a weight row (one block, one
//     scale) straight into the f16 LDS tile with the same function as the
//     standalone dequant, so no separate dequant pass or f16 copy exists.
//   * Strata PR #109 ("Measured"): results must not depend on a split of the
//     reduction; there is no split-k here.
// Tiles are chosen for 64-wide wavefronts: each wave owns (TM/WM) x (TN/WN)
// of 32x32 MFMA blocks; A/W k-tiles go global -> registers -> LDS (double
// buffered, XOR-swizzled 16-byte chunks so each MFMA operand read is
// bank-conflict free), one barrier per k-tile.
#include "device_common.h"
#include "internal.h"

namespace skinny {

namespace {

constexpr int kBK = 32;        // k per LDS tile: two 32x32x16 MFMA steps
constexpr int kCPR = kBK / 8;  // 16-byte chunks per tile row

// chunk c of tile row r lives at chunk (c ^ swz(r)); eight consecutive rows
// read at the same logical chunk then hit eight different 16-byte bank groups
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 3; }

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
  // Q8_0 rows arrive as two 16-code halves per k-tile; f16/bf16 rows as four chunks
  constexpr int B_UNITS = (WK == WK_Q8) ? TN * 2 : TN * kCPR;
  constexpr int B_ITERS = (B_UNITS + NT - 1) / NT;

  __shared__ u32x4 sA[2][A_CHUNKS];
  __shared__ u32x4 sB[2][TN * kCPR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid / WN;
  const int wn = wid - wm * WN;

  const int64_t tiles_n = (g.N + TN - 1) / TN;
  const int64_t bm = blockIdx.x / tiles_n;
  const int64_t bn = blockIdx.x - bm * tiles_n;
  const int64_t row0 = bm * TM;
  const int64_t col0 = bn * TN;

  const uint16_t* __restrict__ A = g.A;
  const int64_t K = g.K;
  const int nk = (int)((K + kBK - 1) / kBK);

  u32x4 ra[A_ITERS];
  u32x4 rb[B_ITERS];
  uint16_t rs[B_ITERS];  // Q8_0 scale of each staged half-row

  auto load_tiles = [&](int kt) {
    const int64_t k0 = (int64_t)kt * kBK;
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      const int q = tid + i * NT;
      const int r = q / kCPR;
      const int c = q - r * kCPR;
      const int64_t gr = row0 + r;
      const int64_t kc = k0 + c * 8;
      const bool ok = (q < A_CHUNKS) && gr < g.M && kc < K;
      ra[i] = ok ? *(const u32x4*)(A + gr * g.lda + kc) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      const int q = tid + i * NT;
      if constexpr (WK == WK_Q8) {
        const int r = q >> 1;
        const int h = q & 1;
        const int64_t gr = col0 + r;
        const bool ok = (q < B_UNITS) && gr < g.N;  // K % 32 == 0, so k0 < K covers the row
        const int8_t* wq = (const int8_t*)g.W;
        rb[i] = ok ? *(const u32x4*)(wq + gr * K + k0 + h * 16) : u32x4{0u, 0u, 0u, 0u};
        rs[i] = ok ? g.scales[gr * (K >> 5) + (k0 >> 5)] : (uint16_t)0;
      } else {
        const int r = q / kCPR;
        const int c = q - r * kCPR;
        const int64_t gr = col0 + r;
        const int64_t kc = k0 + c * 8;
        const bool ok = (q < B_UNITS) && gr < g.N && kc < K;
        const uint16_t* w16 = (const uint16_t*)g.W;
        rb[i] = ok ? *(const u32x4*)(w16 + gr * K + kc) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
      const int q = tid + i * NT;
      if (q < A_CHUNKS) {
        const int r = q / kCPR;
        const int c = q - r * kCPR;
        sA[buf][r * kCPR + (c ^ swz(r))] = ra[i];
      }
    }
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
      const int q = tid + i * NT;
      if (q < B_UNITS) {
        if constexpr (WK == WK_Q8) {
          const int r = q >> 1;
          const int h = q & 1;
          const _Float16 d = half_from_bits(rs[i]);
          const u32x4 codes = rb[i];
          const u32x2 lo = {(uint32_t)codes[0], (uint32_t)codes[1]};
          const u32x2 hi = {(uint32_t)codes[2], (uint32_t)codes[3]};
          sB[buf][r * kCPR + ((2 * h) ^ swz(r))] = q8_dequant8(lo, d);
          sB[buf][r * kCPR + ((2 * h + 1) ^ swz(r))] = q8_dequant8(hi, d);
        } else {
          const int r = q / kCPR;
          const int c = q - r * kCPR;
          sB[buf][r * kCPR + (c ^ swz(r))] = rb[i];
        }
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

  load_tiles(0);
  store_tiles(0);
  __syncthreads();

  const int lrow = lane & 31;
  const int lk = lane >> 5;  // which 8-wide half of an MFMA k-step this lane feeds

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int c = ks * 2 + lk;
      u32x4 af[FM];
      u32x4 bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 32 + lrow;
        af[i] = sA[cur][r * kCPR + (c ^ swz(r))];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 32 + lrow;
        bf[j] = sB[cur][r * kCPR + (c ^ swz(r))];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma32<WK>(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

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
      make_tile<256, 128, 2, 2>("256x128_w2x2"),
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

constexpr int kTileCount = 9;

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
