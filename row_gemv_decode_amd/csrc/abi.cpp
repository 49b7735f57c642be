// abi.cpp -- the C ABI declared in include/skinny.h: argument validation (all
// on the host, before any HIP call), the plan (GEMV split and GEMM tile
// selection) and dispatch to the kernels in gemv.hip / gemm.hip.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>

#include "internal.h"
#include "skinny.h"

using namespace skinny;

static_assert(SKINNY_STATIC_SCRATCH_BYTES == kStaticScratchBytes, "static scratch size");
static_assert(SKINNY_STATIC_COUNTER_BYTES == kStaticCounterBytes, "static counter region");

struct skinny_plan {
  skinny_mm_desc d;   // normalised copy (lda/ldc filled in)
  int num_cus;
  int w_kind;         // WK_*
  int c_kind;         // CK_*
  // GEMV work split, a function of k only (row invariance across m)
  int gemv_T;
  int gemv_S;
  // GEMV columns per wave: gemv_cpw from n, S and the CU count (the
  // arrival counters of a k split across workgroups are laid out by it), and
  // the launch shape each m uses, gemv_cpw_m[m] (a column's arithmetic does not
  // depend on how many columns a wave owns, so it may change with m)
  int gemv_cpw;
  int gemv_cpw_m[kGemvMaxM + 1];
  // GEMM k split (ranges of gemm_kps k-tiles), a function of n, k and the CU
  // count only (M-invariance within the plan)
  int gemm_splits;
  int gemm_kps;
};

namespace {

bool log_enabled() {
  static const int on = [] {
    const char* s = std::getenv("SKINNY_LOG");
    return (s != nullptr && s[0] == '1') ? 1 : 0;
  }();
  return on != 0;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int to_wkind(int dt) {
  return dt == SKINNY_F16    ? WK_F16
         : dt == SKINNY_BF16  ? WK_BF16
         : dt == SKINNY_Q8_0  ? WK_Q8
         : dt == SKINNY_Q4_0  ? WK_Q4
                              : WK_Q2;
}

bool block_quantised(int dt) { return dt == SKINNY_Q8_0 || dt == SKINNY_Q4_0 || dt == SKINNY_Q2_0; }
int to_ckind(int dt) { return dt == SKINNY_F32 ? CK_F32 : dt == SKINNY_F16 ? CK_F16 : CK_BF16; }

// k split of the GEMV: each wave covers 64*T chunks of eight elements; T in
// {1, 2} (registers hold T * m * 16 bytes of A per lane).  Depends on k only.
void gemv_split(int64_t k, int* T_out, int* S_out) {
  const int64_t nchunks = k / 8;
  // candidates (T = 2 first, so it wins ties): the fewest idle chunk slots,
  // preferring splits that one workgroup can sum
  struct Cand {
    int T;
    int64_t S;
  } cand[2] = {{2, (nchunks + 127) / 128}, {1, (nchunks + 63) / 64}};
  int best = 0;
  for (int i = 1; i < 2; ++i) {
    const bool in_i = cand[i].S <= kGemvBlockSplitMax, in_b = cand[best].S <= kGemvBlockSplitMax;
    const int64_t waste_i = cand[i].S * 64 * cand[i].T - nchunks;
    const int64_t waste_b = cand[best].S * 64 * cand[best].T - nchunks;
    if ((in_i && !in_b) || (in_i == in_b && waste_i < waste_b)) best = i;
  }
  *T_out = cand[best].T;
  *S_out = (int)cand[best].S;
}

// columns per wave: enough for about `waves_per_cu` waves per CU, but at
// most kGemvCpwMax columns so the wave's weight loads all fit in registers;
// a power of two (the kernels are compiled for 1, 2, 4 and 8)
int gemv_cols_per_wave(int64_t n, int S, int num_cus, int waves_per_cu) {
  const int64_t target_waves = (int64_t)waves_per_cu * num_cus;
  const int64_t want = (n * S) / (target_waves > 0 ? target_waves : 1);
  int cpw = 1;
  while (cpw * 2 <= want && cpw * 2 <= kGemvCpwMax) cpw *= 2;
  return cpw;
}

// GEMM k split: narrow N leaves most CUs idle at moderate M, so the plan
// also holds a k split, used at the m where the cost model prefers it: k is cut
// until the column tiles (of 64) times the splits reach an eighth of the CU
// count (32 on 256 CUs), keeping at least four 64-wide k-tiles per split and
// at most four splits, with an even number of k-tiles per split.  Depends on
// n, k and the CU count only.  Four was the best chunk count measured on
// MI355X for N = 96, K = 2560 over M = 512 .. 2048 (best tile and launch shape
// per M, summed: 10 chunks 59.9 us, 5 57.0, 4 55.4, 3 57.5): fewer, longer
// chunks cost less fixed time per block and fewer partial sums to add.
void gemm_split(int64_t n, int64_t k, int num_cus, int* splits, int* kps) {
  const int64_t nk = (k + 63) / 64;
  const int64_t col_tiles = (n + 63) / 64;
  int64_t target = num_cus / 8;
  if (target < 8) target = 8;
  int64_t s = (target + col_tiles - 1) / col_tiles;
  if (s > nk / 4) s = nk / 4;
  if (s > 4) s = 4;
  if (s < 1) s = 1;
  int64_t per = (nk + s - 1) / s;
  if (per % 2 != 0 && per < nk) ++per;  // even chunks: a chunked launch folds between tile pairs
  *kps = (int)per;
  *splits = (int)((nk + per - 1) / per);
}

bool use_gemv(const skinny_plan* p, int64_t m) {
  if (p->d.flags & SKINNY_FORCE_GEMV) return true;
  if (p->d.flags & SKINNY_FORCE_GEMM) return false;
  return m <= kGemvMaxM;
}

// GEMM tile selector (opus r35 track A, section 2: the tile is chosen per
// M, and a tile whose last row-block is mostly padding loses -- a 128-row
// tile loses whenever M % 128 is 1..64).  Here the choice comes from a cost
// model fitted to MI355X measurements of every tile (K = 2560, N = 96 and
// 7680, M = 150 .. 2048, cold weights):
//   t      time of one block per 64-wide k-tile when it runs alone (us)
//   c      blocks of the tile one CU holds at once (LDS)
//   a      slow-down when the whole machine is busy: a round with b of its
//          CUs * c slots filled runs 1 + a * b / (CUs * c) times slower
//   sigma  slow-down of a round in which some CU holds two blocks
// est = k-tiles per block * t * sum over rounds of round factors, with
// rounds of CUs * c blocks.  Padded blocks count in full, which is what makes
// a half-padded tail tile lose.
struct TileCost {
  double t;
  int c;
  double a;
  double sigma;
};

constexpr int kCostRows = 18;  // must equal gemm_tile_count(); the plan checks it

const TileCost& tile_cost(int id) {
  // indexed like the tile table in gemm.hip
  static const TileCost kCost[] = {
      {1.7098, 1, 0.280, 1.000},  // 256x256_w2x2
      {1.4204, 1, 0.360, 1.000},  // 256x256_w2x4
      {0.8404, 1, 0.320, 1.000},  // 256x128_w4x2
      {1.0466, 1, 0.240, 1.000},  // 256x128_w2x2
      {1.0163, 1, 0.280, 1.000},  // 128x256_w2x2
      {0.5247, 1, 0.440, 1.000},  // 128x128_w2x2
      {0.4307, 2, 0.400, 1.425},  // 128x64_w2x2
      {0.4411, 2, 0.900, 1.175},  // 64x128_w2x2
      {0.2888, 2, 0.000, 2.175},  // 64x64_w2x2
      {0.4583, 1, 0.340, 1.000},  // 128x96_w4x1
      {0.5776, 2, 0.120, 1.225},  // 64x96_w2x1
      {0.3722, 1, 0.000, 1.000},  // 32x96_w1x1
      {0.2406, 2, 0.400, 1.000},  // 32x64_w1x2
      {0.8760, 1, 0.080, 1.000},  // 192x128_w2x2
      {1.4250, 1, 0.000, 1.000},  // 192x256_w2x4
      {1.1030, 1, 0.145, 1.000},  // 192x192_w3x2
      {0.2700, 2, 0.000, 2.000},  // 32x32_w1x1
      {0.8000, 1, 0.080, 1.000},  // 192x96_w6x1
  };
  static_assert(sizeof(kCost) / sizeof(kCost[0]) == kCostRows, "one cost row per tile");
  return kCost[id];
}

// estimated time of tile `id` at m rows when each of its blocks is repeated
// `copies` times along k and covers `ktiles` 64-wide k-tiles
double tile_estimate(const skinny_plan* p, int id, int64_t m, int64_t copies, int64_t ktiles) {
  const GemmTileInfo& t = gemm_tile(id);
  const TileCost& tc = tile_cost(id);
  const int64_t blocks = ((m + t.tm - 1) / t.tm) * ((p->d.n + t.tn - 1) / t.tn) * copies;
  const int64_t cus = p->num_cus;
  const int64_t slots = cus * tc.c;
  double rounds = 0.0;
  // sigma was fitted on blocks of 40 k-tiles; two short blocks on one CU mostly
  // overlap their fixed latencies, so the penalty shrinks with the block
  const double short_block = ktiles < 40 ? (double)ktiles / 40.0 : 1.0;
  const double sigma = 1.0 + (tc.sigma - 1.0) * short_block;
  for (int64_t left = blocks; left > 0; left -= slots) {
    const int64_t nb = left < slots ? left : slots;
    const int64_t busiest = (nb + cus - 1) / cus;  // blocks on the busiest CU
    rounds += (busiest >= 2 ? sigma : 1.0) * (1.0 + tc.a * (double)nb / (double)slots);
  }
  // block-quantised weights are dequantised per fragment: about 1.65x the
  // f16 time per k-tile on MI355X (measured for Q8_0; Q4_0 and Q2_0 taken
  // the same)
  const double kind = (p->w_kind == WK_Q8 || p->w_kind == WK_Q4 || p->w_kind == WK_Q2) ? 1.65 : 1.0;
  return (double)ktiles * tc.t * kind * rounds;
}

// the split launch's extra cost, fitted to MI355X runs (N = 96 and 512,
// K = 2560, four chunks of ten k-tiles): about 4.5 us for the blocks' fixed
// costs and the reduce launch, plus the fp32 partials written and read back
// at about 2 TB/s
double reduce_estimate(const skinny_plan* p, int64_t m) {
  const double bytes = (double)(p->gemm_splits + 1) * (double)m * (double)p->d.n * 4.0;
  return 4.5 + bytes / 2.0e6;
}

struct GemmChoice {
  int tile;
  int shape;   // kGemmPlain, kGemmChunked (in-block chunk fold) or kGemmFold (last block folds)
  bool split;  // one block per (tile, chunk): the plain shape + the reduce launch, or the fold shape
  double est;
};

// The fold launch (one block per (tile, chunk); the last block of a tile to
// finish adds the tile's chunk sums in order) gives the split launch's bits
// without the reduce launch, but measured slower than split + reduce on every
// MI355X shape tried (N = 96 and 512, K = 2560, M = 306 .. 2048: e.g. 13.6
// against 7.5 us at N = 96, M = 512 on 64 x 64 tiles): one block per tile
// reads all of the tile's chunk sums after a device-scope handoff, where
// the reduce launch spreads them over every CU.  So a plan takes it only
// when SKINNY_GEMM_FOLD_LAUNCH asks for it.
GemmChoice choose_gemm(const skinny_plan* p, int64_t m) {
  const int64_t nk = (p->d.k + 63) / 64;
  const int C = p->gemm_splits;
  GemmChoice best{0, kGemmPlain, false, 0.0};
  bool have = false;
  const int first = p->d.tile_id >= 0 ? p->d.tile_id : 0;
  const int last = p->d.tile_id >= 0 ? p->d.tile_id + 1 : gemm_tile_count();
  for (int id = first; id < last; ++id) {
    GemmChoice c[2];
    int n = 0;
    if (C == 1) {
      c[n++] = GemmChoice{id, kGemmPlain, false, tile_estimate(p, id, m, 1, nk)};
    } else if ((p->d.flags & SKINNY_GEMM_FOLD_LAUNCH) && gemm_tile_foldable(id)) {
      c[n++] = GemmChoice{id, kGemmFold, true, tile_estimate(p, id, m, C, p->gemm_kps)};
    } else {
      const bool force_one = (p->d.flags & SKINNY_GEMM_ONE_LAUNCH) != 0;
      const bool force_split = (p->d.flags & (SKINNY_GEMM_SPLIT_LAUNCH | SKINNY_GEMM_FOLD_LAUNCH)) != 0;
      const bool one_ok = gemm_tile_chunkable(id) && !force_split;
      const bool split_ok = !force_one || !gemm_tile_chunkable(id);
      if (split_ok)
        c[n++] = GemmChoice{id, kGemmPlain, true,
                            tile_estimate(p, id, m, C, p->gemm_kps) + reduce_estimate(p, m)};
      if (one_ok) c[n++] = GemmChoice{id, kGemmChunked, false, tile_estimate(p, id, m, 1, nk)};
    }
    for (int i = 0; i < n; ++i) {
      if (!have || c[i].est < best.est * (1.0 - 1e-9)) {
        best = c[i];
        have = true;
      }
    }
  }
  return best;
}

// Workspace: [one arrival counter per GEMV column range, when the GEMV's k
// splits are summed across workgroups] [fp32 partial sums: the GEMV's
// S x m x n in that case, or the GEMM's splits x m x n when the GEMM splits
// k].  The counters come first so GEMM partials never overwrite them; they
// must be zero before the first call and every call leaves them at zero.
// Partial sums need no initial value.
constexpr size_t kWsAlign = 256;

size_t round_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool gemv_global_split(const skinny_plan* p) { return p->gemv_S > kGemvBlockSplitMax; }

// column ranges (waves per k split) of the launch for m rows
int64_t gemv_waves_per_split(const skinny_plan* p, int64_t m) {
  const int cpw = p->gemv_cpw_m[m < kGemvMaxM ? m : kGemvMaxM];
  return (p->d.n + cpw - 1) / cpw;
}

size_t gemv_counter_bytes(const skinny_plan* p) {
  return gemv_global_split(p)
             ? round_up((size_t)((p->d.n + p->gemv_cpw - 1) / p->gemv_cpw) * sizeof(uint32_t))
             : 0;
}

bool plan_may_gemm(const skinny_plan* p) {
  return !(p->d.flags & SKINNY_FORCE_GEMV) && (p->d.max_m > kGemvMaxM || (p->d.flags & SKINNY_FORCE_GEMM));
}

bool plan_may_fold(const skinny_plan* p) {
  return plan_may_gemm(p) && p->gemm_splits > 1 && (p->d.flags & SKINNY_GEMM_FOLD_LAUNCH);
}

int64_t tile_count(int id, int64_t m, int64_t n) {
  const GemmTileInfo& t = gemm_tile(id);
  return ((m + t.tm - 1) / t.tm) * ((n + t.tn - 1) / t.tn);
}

// the fold launch's largest tile count (one arrival counter each) and chunk
// sums (TM x TN fp32 per tile and chunk) over the tiles it may run, at max_m
size_t fold_counter_bytes_max(const skinny_plan* p) {
  if (!plan_may_fold(p)) return 0;
  int64_t most = 0;
  for (int id = 0; id < gemm_tile_count(); ++id)
    if (gemm_tile_foldable(id) && (p->d.tile_id < 0 || p->d.tile_id == id)) {
      const int64_t t = tile_count(id, p->d.max_m, p->d.n);
      most = t > most ? t : most;
    }
  return round_up((size_t)most * sizeof(uint32_t));
}

size_t fold_slot_bytes(int id, int64_t m, const skinny_plan* p) {
  const GemmTileInfo& t = gemm_tile(id);
  return round_up((size_t)tile_count(id, m, p->d.n) * (size_t)p->gemm_splits * (size_t)t.tm * (size_t)t.tn *
                  sizeof(float));
}

// the counter region: the GEMV's arrival counters or the fold launch's
size_t counter_bytes(const skinny_plan* p) {
  const size_t a = gemv_counter_bytes(p), b = fold_counter_bytes_max(p);
  return a > b ? a : b;
}

size_t gemv_partial_bytes(const skinny_plan* p, int64_t m) {
  return gemv_global_split(p)
             ? round_up((size_t)p->gemv_S * (size_t)m * (size_t)p->d.n * sizeof(float))
             : 0;
}

size_t gemm_partial_bytes(const skinny_plan* p, int64_t m) {
  const GemmChoice gc = choose_gemm(p, m);
  if (!gc.split) return 0;
  if (gc.shape == kGemmFold) return fold_slot_bytes(gc.tile, m, p);
  return round_up((size_t)p->gemm_splits * (size_t)m * (size_t)p->d.n * sizeof(float));
}

// fp32 rows of A: the GEMV rounds them to bf16 as it loads them (one
// launch).  A wave then holds twice the A bytes in flight per row, which
// measured slower than a separate cast launch once A is not staged in LDS
// (k split, S > 1) and m > 10 (n = 1, 256, 2048 at k = 2048..16384); there
// the run casts the rows into the workspace and the bf16 GEMV reads them.
// Both shapes round with the same conversion and sum identically, so the
// choice per m changes no bit.
constexpr int64_t kA32FusedMaxM = 10;

int64_t gemv_row_groups(const skinny_plan* p, int64_t m);

bool a32_cast_first(const skinny_plan* p, int64_t m) {
  return p->d.a_dtype == SKINNY_F32 && p->gemv_S > 1 && m > kA32FusedMaxM && gemv_row_groups(p, m) == 1;
}

// elements of A a cast-first run converts: rows 0..m-1 at stride lda, the
// last one only up to k
int64_t a32_cast_count(const skinny_plan* p, int64_t m) { return (m - 1) * p->d.lda + p->d.k; }

// A run's scratch is two regions: the arrival counters (zero between runs;
// every run leaves them at zero) and the data region, which needs no initial
// value: the partial sums (the GEMV's S x m x n, or the GEMM's chunks x m x n)
// and after them the cast rows of a cast-first run.
struct Scratch {
  uint32_t* counters;
  char* data;
};

// bytes of the data region before the cast rows: partial sums
size_t partial_bytes_for(const skinny_plan* p, int64_t m) {
  return use_gemv(p, m) ? gemv_partial_bytes(p, m) : gemm_partial_bytes(p, m);
}

// bytes of the data region a run at m rows needs (with or without the top-k)
size_t data_bytes_for(const skinny_plan* p, int64_t m) {
  const size_t a16 = a32_cast_first(p, m) ? round_up((size_t)a32_cast_count(p, m) * 2) : 0;
  return partial_bytes_for(p, m) + a16;
}

// bytes of a caller's workspace a run at m rows needs: [counters][data], or
// nothing when the run needs no data region (counters exist only beside
// partial sums)
size_t workspace_bytes_for(const skinny_plan* p, int64_t m) {
  const size_t data = data_bytes_for(p, m);
  return data > 0 ? counter_bytes(p) + data : 0;
}

// the two regions inside a caller's workspace
Scratch caller_scratch(const skinny_plan* p, void* workspace) {
  char* ws = (char*)workspace;
  return Scratch{(uint32_t*)ws, ws != nullptr ? ws + counter_bytes(p) : nullptr};
}

skinny_status hip_status(hipError_t e) { return e == hipSuccess ? SKINNY_OK : SKINNY_ERR_HIP; }

// the GEMV launch for m rows runs the kernel for gemv_kernel_rows(p, m) rows
// in gemv_row_groups(p, m) workgroup rows
int64_t gemv_kernel_rows(const skinny_plan* p, int64_t m) { return m / gemv_row_groups(p, m); }

GemvArgs gemv_args(const skinny_plan* p, int64_t m_rows, const void* A, const void* W, const void* scales,
                   void* C, int64_t ldc, const Scratch& sc) {
  const int64_t m = gemv_kernel_rows(p, m_rows);
  GemvArgs g;
  g.row_groups = (int32_t)gemv_row_groups(p, m_rows);
  // wave w of an in-block split workgroup: range w / S, split w % S
  g.wave_range = 0;
  g.wave_split = 0;
  if (p->gemv_S <= kGemvBlockSplitMax)
    for (int w = 0; w < kGemvMaxWavesPerBlock; ++w) {
      g.wave_range |= (uint32_t)(w / p->gemv_S) << (4 * w);
      g.wave_split |= (uint32_t)(w % p->gemv_S) << (4 * w);
    }
  g.A = A;
  g.a_kind = p->d.a_dtype == SKINNY_F32 ? kAF32 : kA16;
  g.lda = p->d.lda;
  g.W = W;
  g.scales = (const uint16_t*)scales;
  g.n = p->d.n;
  g.k = p->d.k;
  g.nchunks = (int32_t)(p->d.k / 8);
  g.S = p->gemv_S;
  g.cpw = p->gemv_cpw_m[m < kGemvMaxM ? m : kGemvMaxM];
  g.waves_per_split = (int32_t)gemv_waves_per_split(p, m);
  g.cg_per_block = 0;
  g.C = C;
  g.ldc = ldc;
  g.epilogue = (p->d.flags & SKINNY_EPILOGUE_SIGMOID) ? kEpiSigmoid : kEpiNone;
  g.counters = gemv_global_split(p) ? sc.counters : nullptr;
  g.partial = gemv_global_split(p) ? (float*)sc.data : nullptr;
  return g;
}

GemmArgs gemm_args(const skinny_plan* p, int64_t m, const void* A, const void* W,
                   const void* scales, void* C, int64_t ldc, const Scratch& sc) {
  GemmArgs g;
  g.A = (const uint16_t*)A;
  g.lda = p->d.lda;
  g.W = W;
  g.scales = (const uint16_t*)scales;
  g.M = m;
  g.N = p->d.n;
  g.K = p->d.k;
  g.C = C;
  g.ldc = ldc;
  g.splits = 1;
  g.kt_per_split = p->gemm_kps;
  g.partial = p->gemm_splits > 1 ? (float*)sc.data : nullptr;
  g.counters = sc.counters;
  return g;
}

// checks shared by the run calls (everything but the workspace)
skinny_status check_run_args(const skinny_plan* p, int64_t m, const void* A, const void* W,
                             const void* scales, const void* C) {
  if (p == nullptr) return SKINNY_ERR_INVALID_ARG;
  if (m < 1 || m > p->d.max_m) return SKINNY_ERR_INVALID_ARG;
  if (A == nullptr || W == nullptr || C == nullptr) return SKINNY_ERR_INVALID_ARG;
  const bool qb = block_quantised(p->d.w_dtype);
  if (qb != (scales != nullptr)) return SKINNY_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(W) || !aligned16(C) || (qb && !aligned16(scales)))
    return SKINNY_ERR_ALIGNMENT;
  // the GEMV numbers its waves (k splits x column ranges of one row group) in
  // 32 bits
  if (use_gemv(p, m) && gemv_waves_per_split(p, gemv_kernel_rows(p, m)) * p->gemv_S > (1LL << 31) - 1024)
    return SKINNY_ERR_SHAPE;
  return SKINNY_OK;
}

// the argument checks plus the caller's workspace
skinny_status check_run(const skinny_plan* p, int64_t m, const void* A, const void* W,
                        const void* scales, const void* C, const void* workspace,
                        size_t workspace_bytes) {
  const skinny_status st = check_run_args(p, m, A, W, scales, C);
  if (st != SKINNY_OK) return st;
  const size_t need = workspace_bytes_for(p, m);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return SKINNY_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SKINNY_ERR_ALIGNMENT;
  }
  return SKINNY_OK;
}

// GEMV workgroup shape.  Splits summed inside a workgroup: S waves per column
// range and as many ranges as fit in kGemvMaxWavesPerBlock waves.  Without a
// split (or with splits summed across workgroups) 4 waves spread the work over
// the most CUs.
struct GemvBlock {
  int waves;
  int ranges;  // column ranges per workgroup (splits summed inside), else 0
};

GemvBlock gemv_block(const skinny_plan* p) {
  const int S = p->gemv_S;
  const int plain = 4;
  if (S == 1) return {plain, plain};
  if (S <= kGemvBlockSplitMax) {
    const int ranges = kGemvMaxWavesPerBlock / S;
    return {ranges * S, ranges};
  }
  return {plain, 0};
}

int64_t gemv_blocks(const skinny_plan* p, const GemvBlock& b, int64_t m) {
  const int64_t wps = gemv_waves_per_split(p, m);
  if (b.ranges > 0) return (wps + b.ranges - 1) / b.ranges;
  return (wps * p->gemv_S + b.waves - 1) / b.waves;
}

// Row groups.  The launch for m rows may run the kernel for r rows (r
// divides m) in m / r workgroup rows (blockIdx.y), row group y taking rows
// y r .. y r + r - 1 of A and C.  Rows are independent and a row's
// arithmetic does not depend on how many rows its kernel holds, so this
// changes no bit; it trades re-reads of the weight (from L2 or the
// last-level cache) for more workgroups and fewer rows per wave.  Never with
// k split across workgroups.  Two cases, measured on MI355X (graph replay,
// cold weights):
//   - a few workgroups: when the one-row grid times m fits in half the CUs
//     (the scalar gate: n = 1, one workgroup), r = 1 -- 2.19 / 3.88 / 6.12
//     -> 2.23 / 2.60 / 2.60 us at m = 1 / 8 / 16;
//   - unsplit k: the smallest power-of-two r whose m / r groups keep the
//     launch within about ten waves per CU -- n x k = 608 x 896: 2.59 /
//     3.10 / 3.86 -> 2.35 / 2.66 / 3.31 us at m = 4 / 8 / 16 (r = 1 / 2 / 4);
//     at 4864 x 896 no r fits, and every r measured slower there.
int64_t gemv_row_groups(const skinny_plan* p, int64_t m) {
  if (m <= 1 || gemv_global_split(p)) return 1;
  if (gemv_blocks(p, gemv_block(p), 1) * m <= p->num_cus / 2) return m;
  if (p->gemv_S == 1) {
    for (int64_t r = 1; r < m; r *= 2)
      if (m % r == 0 && gemv_waves_per_split(p, r) * (m / r) <= 10 * (int64_t)p->num_cus) return m / r;
  }
  return 1;
}

// enqueue C = A . W for m rows, then (when idx/val are given) the top-k launch
// over the rows of C (Strata PR #109, "What": one multi-row GEMV launch and
// one multi-row top-10 launch per window)
skinny_status enqueue_mm(const skinny_plan* p, int64_t m, const void* A, const void* W,
                         const void* scales, void* C, int64_t ldc, int c_kind, const Scratch& sc,
                         int32_t* topk_idx, float* topk_val, int32_t topk, hipStream_t stream) {
  const bool want_topk = topk_idx != nullptr;
  if (use_gemv(p, m)) {
    GemvArgs g = gemv_args(p, m, A, W, scales, C, ldc, sc);
    const int64_t mk = gemv_kernel_rows(p, m);
    const GemvBlock b = gemv_block(p);
    g.cg_per_block = b.ranges;
    if (a32_cast_first(p, m)) {
      uint16_t* a16 = (uint16_t*)(sc.data + partial_bytes_for(p, m));
      skinny_status st = hip_status(launch_cast_f32_bf16(a32_cast_count(p, m), (const float*)A, a16, stream));
      if (st != SKINNY_OK) return st;
      g.A = a16;
      g.a_kind = kA16;
    }
    skinny_status st = hip_status(launch_gemv(g, (int)mk, p->gemv_T, p->w_kind, c_kind, b.waves, stream));
    if (st != SKINNY_OK || !want_topk) return st;
    return hip_status(launch_topk((const float*)C, (int)m, p->d.n, ldc, topk_idx, topk_val, topk, stream));
  }
  GemmArgs g = gemm_args(p, m, A, W, scales, C, ldc, sc);
  const GemmChoice gc = choose_gemm(p, m);
  if (gc.split) g.splits = p->gemm_splits;
  skinny_status st = hip_status(launch_gemm(gc.tile, g, p->w_kind, c_kind, gc.shape, stream));
  if (st == SKINNY_OK && gc.split && gc.shape == kGemmPlain)
    st = hip_status(launch_splitk_reduce(g, c_kind, stream));
  if (st != SKINNY_OK || !want_topk) return st;
  return hip_status(launch_topk((const float*)C, (int)m, p->d.n, ldc, topk_idx, topk_val, topk, stream));
}

}  // namespace

extern "C" {

int32_t skinny_abi_version(void) { return SKINNY_ABI_VERSION; }

const char* skinny_status_string(skinny_status s) {
  switch (s) {
    case SKINNY_OK: return "ok";
    case SKINNY_ERR_INVALID_ARG: return "invalid argument";
    case SKINNY_ERR_UNSUPPORTED: return "unsupported dtype combination or flag";
    case SKINNY_ERR_ALIGNMENT: return "pointer or stride misaligned";
    case SKINNY_ERR_SHAPE: return "unsupported shape";
    case SKINNY_ERR_HIP: return "HIP runtime error";
    case SKINNY_ERR_WORKSPACE: return "workspace missing or too small";
    case SKINNY_ERR_SCRATCH: return "run needs more scratch than the library's static array holds";
  }
  return "unknown status";
}

int32_t skinny_gemm_tile_count(void) { return gemm_tile_count(); }

const char* skinny_gemm_tile_name(int32_t tile_id) {
  if (tile_id < 0 || tile_id >= gemm_tile_count()) return nullptr;
  return gemm_tile(tile_id).name;
}

skinny_status skinny_mm_plan(const skinny_mm_desc* desc, skinny_plan** out_plan) {
  if (desc == nullptr || out_plan == nullptr) return SKINNY_ERR_INVALID_ARG;
  if (desc->struct_size < sizeof(skinny_mm_desc)) return SKINNY_ERR_INVALID_ARG;
  skinny_mm_desc d = *desc;

  if (d.a_dtype != SKINNY_F16 && d.a_dtype != SKINNY_BF16 && d.a_dtype != SKINNY_F32)
    return SKINNY_ERR_UNSUPPORTED;
  // fp32 rows are rounded to bf16 as the GEMV loads them: bf16 weights, GEMV
  // regime only
  if (d.a_dtype == SKINNY_F32 &&
      (d.w_dtype != SKINNY_BF16 || d.max_m > kGemvMaxM || (d.flags & SKINNY_FORCE_GEMM)))
    return SKINNY_ERR_UNSUPPORTED;
  if (d.a_dtype == SKINNY_F16 && d.w_dtype != SKINNY_F16 && !block_quantised(d.w_dtype))
    return SKINNY_ERR_UNSUPPORTED;
  if (d.a_dtype == SKINNY_BF16 && d.w_dtype != SKINNY_BF16) return SKINNY_ERR_UNSUPPORTED;
  if (d.c_dtype != SKINNY_F32 && d.c_dtype != SKINNY_F16 && d.c_dtype != SKINNY_BF16)
    return SKINNY_ERR_UNSUPPORTED;
  if (d.max_m < 1 || d.n < 1 || d.k < 8) return SKINNY_ERR_INVALID_ARG;
  if (d.max_m > (1LL << 31) - 1 || d.n > (1LL << 31) - 1 || d.k > (1LL << 31) - 1)
    return SKINNY_ERR_INVALID_ARG;
  if (d.k % 8 != 0) return SKINNY_ERR_SHAPE;
  if (block_quantised(d.w_dtype) && d.k % 32 != 0) return SKINNY_ERR_SHAPE;
  if (d.lda == 0) d.lda = d.k;
  if (d.ldc == 0) d.ldc = d.n;
  if (d.lda < d.k || d.ldc < d.n) return SKINNY_ERR_SHAPE;
  if (d.lda % 8 != 0) return SKINNY_ERR_ALIGNMENT;  // A rows are read 16 bytes at a time
  if (d.flags & ~(SKINNY_FORCE_GEMV | SKINNY_FORCE_GEMM | SKINNY_GEMM_SPLIT_LAUNCH | SKINNY_GEMM_ONE_LAUNCH |
                  SKINNY_GEMM_FOLD_LAUNCH | SKINNY_EPILOGUE_SIGMOID))
    return SKINNY_ERR_UNSUPPORTED;
  // the gate's sigmoid is applied by the GEMV only, for bf16 weights and an
  // f32 or f16 gate
  if ((d.flags & SKINNY_EPILOGUE_SIGMOID) &&
      (d.max_m > kGemvMaxM || (d.flags & SKINNY_FORCE_GEMM) || d.w_dtype != SKINNY_BF16 ||
       d.c_dtype == SKINNY_BF16))
    return SKINNY_ERR_UNSUPPORTED;
  {
    const uint32_t shapes = d.flags & (SKINNY_GEMM_SPLIT_LAUNCH | SKINNY_GEMM_ONE_LAUNCH | SKINNY_GEMM_FOLD_LAUNCH);
    if (shapes & (shapes - 1)) return SKINNY_ERR_INVALID_ARG;  // at most one launch shape forced
  }
  if ((d.flags & SKINNY_FORCE_GEMV) && (d.flags & SKINNY_FORCE_GEMM)) return SKINNY_ERR_INVALID_ARG;
  if ((d.flags & SKINNY_FORCE_GEMV) && d.max_m > kGemvMaxM) return SKINNY_ERR_INVALID_ARG;
  if (gemm_tile_count() != kCostRows) return SKINNY_ERR_UNSUPPORTED;  // a build whose tables disagree
  if (d.tile_id < -1 || d.tile_id >= gemm_tile_count()) return SKINNY_ERR_INVALID_ARG;
  // the GEMM addresses a block's rows through 32-bit buffer offsets
  const bool may_gemm = !(d.flags & SKINNY_FORCE_GEMV) && (d.max_m > kGemvMaxM || (d.flags & SKINNY_FORCE_GEMM));
  if (may_gemm && (d.k > kGemmMaxK || d.lda > kGemmMaxK)) return SKINNY_ERR_SHAPE;
  // the GEMM's k-chunk partials hold up to 16 x max_m x n floats: keep every
  // index and byte count far inside 64 bits
  if (may_gemm && d.max_m > (1LL << 50) / d.n) return SKINNY_ERR_SHAPE;
  // the GEMM fetches a k-tile's two block scales of a row as one 4-byte word,
  // which needs at least two scales per row (k >= 64)
  if (may_gemm && block_quantised(d.w_dtype) && d.k < 64) return SKINNY_ERR_SHAPE;
  if (d.num_cus < 0) return SKINNY_ERR_INVALID_ARG;

  int cus = d.num_cus;
  if (cus == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SKINNY_ERR_HIP;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return SKINNY_ERR_HIP;
    if (cus < 1) return SKINNY_ERR_HIP;
  }

  skinny_plan* p = new (std::nothrow) skinny_plan;
  if (p == nullptr) return SKINNY_ERR_INVALID_ARG;
  p->d = d;
  p->num_cus = cus;
  p->w_kind = to_wkind(d.w_dtype);
  p->c_kind = to_ckind(d.c_dtype);
  gemv_split(d.k, &p->gemv_T, &p->gemv_S);
  // Columns per wave by m (a column's arithmetic does not depend on it).
  // The base is about four waves per CU (it also lays out the arrival
  // counters of a k split across workgroups).  A k split inside the
  // workgroup runs about eight waves per CU.  An unsplit k runs about
  // sixteen waves per CU up to m = 8 and eight above: measured on MI355X at
  // n x k = 4864 x 896 (graph replay, cold weights), one column per wave
  // took 3.64 / 4.12 / 4.69 us at m = 1 / 4 / 8 against 3.72 / 4.39 / 5.17
  // for two, and at m = 16 two columns took 7.00 us against 7.92 for four
  // (more waves hide more of the load and reduction latency).
  p->gemv_cpw = gemv_cols_per_wave(d.n, p->gemv_S, cus, 4);
  for (int m = 0; m <= kGemvMaxM; ++m) {
    if (p->gemv_S == 1)
      p->gemv_cpw_m[m] = gemv_cols_per_wave(d.n, 1, cus, m <= 8 ? 16 : 8);
    else if (p->gemv_S <= kGemvBlockSplitMax)
      p->gemv_cpw_m[m] = gemv_cols_per_wave(d.n, p->gemv_S, cus, 8);
    else
      p->gemv_cpw_m[m] = p->gemv_cpw;
  }
  gemm_split(d.n, d.k, cus, &p->gemm_splits, &p->gemm_kps);
  if (log_enabled()) {
    std::fprintf(stderr, "[skinny] plan n=%lld k=%lld max_m=%lld gemv T=%d S=%d cpw=%d cus=%d\n",
                 (long long)d.n, (long long)d.k, (long long)d.max_m, p->gemv_T, p->gemv_S,
                 p->gemv_cpw, cus);
  }
  *out_plan = p;
  return SKINNY_OK;
}

void skinny_mm_plan_destroy(skinny_plan* plan) { delete plan; }

skinny_status skinny_mm_workspace_size(const skinny_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr) return SKINNY_ERR_INVALID_ARG;
  // the largest need of any run: the GEMV at its largest m, or the GEMM at
  // max_m (each needs the workspace only when it splits k across workgroups)
  // (a GEMM that cuts k into chunks may use the split launch at any m, so
  // its partials are sized for max_m)
  // (the fold launch's chunk sums are TM x TN per tile and chunk: the
  // largest of its tiles at max_m bounds every m)
  size_t need = workspace_bytes_for(plan, plan->d.max_m < kGemvMaxM ? plan->d.max_m : kGemvMaxM);
  if (plan_may_gemm(plan) && plan->gemm_splits > 1) {
    size_t data = round_up((size_t)plan->gemm_splits * (size_t)plan->d.max_m * (size_t)plan->d.n * sizeof(float));
    if (plan_may_fold(plan))
      for (int id = 0; id < gemm_tile_count(); ++id)
        if (gemm_tile_foldable(id) && (plan->d.tile_id < 0 || plan->d.tile_id == id)) {
          const size_t f = fold_slot_bytes(id, plan->d.max_m, plan);
          data = f > data ? f : data;
        }
    const size_t g = counter_bytes(plan) + data;
    need = g > need ? g : need;
  }
  *bytes = need;
  return SKINNY_OK;
}

skinny_status skinny_mm_run(const skinny_plan* plan, int64_t m, const void* A, const void* W,
                            const void* w_scales, void* C, void* workspace,
                            size_t workspace_bytes, void* stream) {
  skinny_status st = check_run(plan, m, A, W, w_scales, C, workspace, workspace_bytes);
  if (st != SKINNY_OK) return st;
  return enqueue_mm(plan, m, A, W, w_scales, C, plan->d.ldc, plan->c_kind, caller_scratch(plan, workspace),
                    nullptr, nullptr, 0, (hipStream_t)stream);
}

skinny_status skinny_mm_run_static(const skinny_plan* plan, int64_t m, const void* A, const void* W,
                                   const void* w_scales, void* C, void* stream) {
  skinny_status st = check_run_args(plan, m, A, W, w_scales, C);
  if (st != SKINNY_OK) return st;
  // sizes first, before any HIP call: the counters must fit their region and
  // the partial sums and cast rows the data region
  const size_t data = data_bytes_for(plan, m);
  if (data > 0 && (counter_bytes(plan) > kStaticCounterBytes || data > kStaticDataBytes))
    return SKINNY_ERR_SCRATCH;
  Scratch sc{nullptr, nullptr};
  if (data > 0) {
    char* base = nullptr;
    st = hip_status(static_scratch((hipStream_t)stream, &base));
    if (st != SKINNY_OK) return st;
    sc = Scratch{(uint32_t*)base, base + kStaticCounterBytes};
  }
  return enqueue_mm(plan, m, A, W, w_scales, C, plan->d.ldc, plan->c_kind, sc, nullptr, nullptr, 0,
                    (hipStream_t)stream);
}

skinny_status gemv_topk_run(const skinny_plan* plan, int64_t m, const void* A, const void* W,
                            const void* w_scales, float* logits, int32_t* topk_idx,
                            float* topk_val, int32_t topk, void* workspace,
                            size_t workspace_bytes, void* stream) {
  skinny_status st = check_run(plan, m, A, W, w_scales, logits, workspace, workspace_bytes);
  if (st != SKINNY_OK) return st;
  if (plan->d.c_dtype != SKINNY_F32 || (plan->d.flags & SKINNY_EPILOGUE_SIGMOID)) return SKINNY_ERR_UNSUPPORTED;
  if (topk_idx == nullptr || topk_val == nullptr) return SKINNY_ERR_INVALID_ARG;
  if (topk < 1 || topk > SKINNY_TOPK_MAX || topk > plan->d.n) return SKINNY_ERR_INVALID_ARG;
  if (!aligned16(topk_idx) || !aligned16(topk_val)) return SKINNY_ERR_ALIGNMENT;
  return enqueue_mm(plan, m, A, W, w_scales, logits, plan->d.ldc, CK_F32, caller_scratch(plan, workspace),
                    topk_idx, topk_val, topk, (hipStream_t)stream);
}

skinny_status skinny_dequant_q2_0_run(int64_t n, int64_t k, const void* qs, const void* d,
                                      void* out, void* stream) {
  if (qs == nullptr || d == nullptr || out == nullptr) return SKINNY_ERR_INVALID_ARG;
  if (n < 1 || k < 32 || n > (1LL << 31) - 1 || k > (1LL << 31) - 1) return SKINNY_ERR_INVALID_ARG;
  if (k % 32 != 0) return SKINNY_ERR_SHAPE;
  if (!aligned16(qs) || !aligned16(d) || !aligned16(out)) return SKINNY_ERR_ALIGNMENT;
  return hip_status(launch_dequant_q2_0(n, k, (const uint8_t*)qs, (const uint16_t*)d, (uint16_t*)out,
                                        (hipStream_t)stream));
}

skinny_status skinny_dequant_q4_0_run(int64_t n, int64_t k, const void* qs, const void* d,
                                      void* out, void* stream) {
  if (qs == nullptr || d == nullptr || out == nullptr) return SKINNY_ERR_INVALID_ARG;
  if (n < 1 || k < 32 || n > (1LL << 31) - 1 || k > (1LL << 31) - 1) return SKINNY_ERR_INVALID_ARG;
  if (k % 32 != 0) return SKINNY_ERR_SHAPE;
  if (!aligned16(qs) || !aligned16(d) || !aligned16(out)) return SKINNY_ERR_ALIGNMENT;
  return hip_status(launch_dequant_q4_0(n, k, (const uint8_t*)qs, (const uint16_t*)d, (uint16_t*)out,
                                        (hipStream_t)stream));
}

skinny_status skinny_dequant_q8_0_run(int64_t n, int64_t k, const void* qs, const void* d,
                                      void* out, void* stream) {
  if (qs == nullptr || d == nullptr || out == nullptr) return SKINNY_ERR_INVALID_ARG;
  if (n < 1 || k < 32 || n > (1LL << 31) - 1 || k > (1LL << 31) - 1) return SKINNY_ERR_INVALID_ARG;
  if (k % 32 != 0) return SKINNY_ERR_SHAPE;
  if (!aligned16(qs) || !aligned16(d) || !aligned16(out)) return SKINNY_ERR_ALIGNMENT;
  return hip_status(launch_dequant_q8_0(n, k, (const int8_t*)qs, (const uint16_t*)d, (uint16_t*)out,
                                        (hipStream_t)stream));
}

skinny_status skinny_cast_f32_bf16_run(int64_t count, const float* in, void* out, void* stream) {
  if (in == nullptr || out == nullptr || count < 1 || count > (1LL << 40)) return SKINNY_ERR_INVALID_ARG;
  const uintptr_t i0 = reinterpret_cast<uintptr_t>(in), o0 = reinterpret_cast<uintptr_t>(out);
  if (i0 < o0 + (uintptr_t)count * 2 && o0 < i0 + (uintptr_t)count * 4) return SKINNY_ERR_INVALID_ARG;
  if (!aligned16(in) || !aligned16(out)) return SKINNY_ERR_ALIGNMENT;
  return hip_status(launch_cast_f32_bf16(count, in, (uint16_t*)out, (hipStream_t)stream));
}

skinny_status skinny_moe_combine_run(int64_t m, int64_t d, int32_t topk, const void* rows, const float* weights,
                                    const void* shared_rows, const float* gate, int32_t rows_dtype, void* out,
                                    int32_t out_dtype, void* stream) {
  if (rows == nullptr || weights == nullptr || out == nullptr) return SKINNY_ERR_INVALID_ARG;
  if ((shared_rows == nullptr) != (gate == nullptr)) return SKINNY_ERR_INVALID_ARG;
  if (m < 1 || m > (1LL << 31) - 1 || d < 8 || d > (1LL << 40) || topk < 1 || topk > SKINNY_TOPK_MAX)
    return SKINNY_ERR_INVALID_ARG;
  // every element index (and byte count) below stays far inside 64 bits
  if (d > (1LL << 56) / (m * (int64_t)topk)) return SKINNY_ERR_INVALID_ARG;
  if (d % 8 != 0) return SKINNY_ERR_SHAPE;
  if ((rows_dtype != SKINNY_F32 && rows_dtype != SKINNY_BF16) || (out_dtype != SKINNY_F32 && out_dtype != SKINNY_BF16))
    return SKINNY_ERR_UNSUPPORTED;
  if (!aligned16(rows) || !aligned16(out) || (shared_rows != nullptr && !aligned16(shared_rows)) ||
      (reinterpret_cast<uintptr_t>(weights) & 3u) != 0 || (reinterpret_cast<uintptr_t>(gate) & 3u) != 0)
    return SKINNY_ERR_ALIGNMENT;
  const uintptr_t in_elem = rows_dtype == SKINNY_F32 ? 4 : 2;
  const uintptr_t o0 = reinterpret_cast<uintptr_t>(out);
  const uintptr_t o1 = o0 + (uintptr_t)m * (uintptr_t)d * (out_dtype == SKINNY_F32 ? 4 : 2);
  auto overlaps = [&](const void* p, uintptr_t bytes) {
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(p);
    return p != nullptr && p0 < o1 && o0 < p0 + bytes;
  };
  if (overlaps(rows, (uintptr_t)m * (uintptr_t)topk * (uintptr_t)d * in_elem) ||
      overlaps(shared_rows, (uintptr_t)m * (uintptr_t)d * in_elem) ||
      overlaps(weights, (uintptr_t)m * (uintptr_t)topk * 4) || overlaps(gate, (uintptr_t)m * 4))
    return SKINNY_ERR_INVALID_ARG;
  CombineArgs a;
  a.m = m;
  a.d = d;
  a.topk = topk;
  a.rows = rows;
  a.weights = weights;
  a.shared = shared_rows;
  a.gate = gate;
  a.out = out;
  const int rk = rows_dtype == SKINNY_F32 ? CK_F32 : CK_BF16;
  const int ok = out_dtype == SKINNY_F32 ? CK_F32 : CK_BF16;
  return hip_status(launch_moe_combine(a, rk, ok, (hipStream_t)stream));
}

skinny_status skinny_mm_plan_info(const skinny_plan* plan, int64_t m, char* buf, size_t len) {
  if (plan == nullptr || buf == nullptr || len == 0) return SKINNY_ERR_INVALID_ARG;
  if (m < 1 || m > plan->d.max_m) return SKINNY_ERR_INVALID_ARG;
  if (use_gemv(plan, m)) {
    // the launch: the kernel for mk rows, in `groups` workgroup rows
    const int64_t mk = gemv_kernel_rows(plan, m);
    const int64_t groups = gemv_row_groups(plan, m);
    const int64_t waves = gemv_waves_per_split(plan, mk) * plan->gemv_S * groups;
    const GemvBlock b = gemv_block(plan);
    char rows_token[40] = "";
    if (groups > 1) std::snprintf(rows_token, sizeof(rows_token), "row_groups=%lld ", (long long)groups);
    std::snprintf(buf, len,
                  "path=gemv m=%lld T=%d S=%d cpw=%d waves=%lld blocks=%lld x %d waves split_reduce=%s "
                  "%s%s%sworkspace=%zu",
                  (long long)m, plan->gemv_T, plan->gemv_S, plan->gemv_cpw_m[mk], (long long)waves,
                  (long long)(gemv_blocks(plan, b, mk) * groups), b.waves,
                  plan->gemv_S == 1 ? "none" : (gemv_global_split(plan) ? "global" : "in-block"), rows_token,
                  plan->d.a_dtype != SKINNY_F32 ? ""
                  : a32_cast_first(plan, m)     ? "a=f32(cast-launch) "
                                                : "a=f32(fused) ",
                  (plan->d.flags & SKINNY_EPILOGUE_SIGMOID) ? "epilogue=sigmoid " : "",
                  workspace_bytes_for(plan, m));
  } else {
    const GemmChoice gc = choose_gemm(plan, m);
    const GemmTileInfo& t = gemm_tile(gc.tile);
    const int64_t blocks =
        ((m + t.tm - 1) / t.tm) * ((plan->d.n + t.tn - 1) / t.tn) * (gc.split ? plan->gemm_splits : 1);
    std::snprintf(buf, len,
                  "path=gemm m=%lld tile=%d name=%s chunks=%d launch=%s blocks=%lld threads=%d "
                  "est_us=%.1f workspace=%zu",
                  (long long)m, gc.tile, t.name, plan->gemm_splits,
                  gc.shape == kGemmFold ? "fold" : gc.split ? "split" : (gc.shape == kGemmChunked ? "one" : "plain"),
                  (long long)blocks,
                  64 * t.wm * t.wn, gc.est, workspace_bytes_for(plan, m));
  }
  return SKINNY_OK;
}

}  // extern "C"
