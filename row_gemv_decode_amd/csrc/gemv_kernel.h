// gemv_kernel.h -- the multi-row GEMV kernel for gfx950 (MI355X), included by
// one translation unit per weight type (gemv_f16.hip, gemv_bf16.hip,
// gemv_q8.hip) and by gemv.hip for the shared wave helpers.
//
// What is computed (the pages print no code for any of it):
//   C[r][j] = sum_kk A[r][kk] * W[j][kk] for r < m <= 16, W stored [n][k]
//   (nx_batchscale_kat: the product must read W once for all m rows, so that
//   us_per_row falls with m; Strata PR #109, "What": the router GEMV reads its
//   weight once for the whole window, with each token's accumulators in
//   exactly the single-token order).
//
// Design (MI355X-first, not the pages' CUDA kernel):
//   * One wavefront owns a k-range of 64*T chunks of eight elements, chunk
//     c = split*64*T + t*64 + lane, and a run of consecutive columns.  Every
//     W load is a coalesced 16-byte load (a wave reads 1 KiB contiguous per
//     instruction); all W loads of the wave are issued before any arithmetic,
//     so the whole weight is in flight at once (the stream is tiny compared
//     with the HBM latency-bandwidth product).
//   * The wave's A slice is loaded once into registers and reused for every
//     column, so the k loop reads no LDS.
//   * Products use v_dot2_f32_{f16,bf16}: two products per lane per
//     instruction into an fp32 accumulator, chunk by chunk in increasing k.
//   * The 64 per-lane partials of each (row, column) are combined by a fixed
//     six-level tree: lanes l ^ 15, l ^ 7 (DPP row mirrors), l ^ 2, l ^ 1 (DPP
//     quad permutes), l ^ 16 and l ^ 32 (v_permlane16/32_swap).  The first
//     levels are "transposed": a lane keeps half of its values and receives
//     the partner's copy of that half, so reducing G columns x M rows costs
//     about 3 * G * M instructions instead of 6 * G * M.  The tree is the same
//     for every value, hence the same for every m.
//   * Nothing in the split, the tree or the per-lane order depends on m, so
//     row r of any call equals the m = 1 call bit for bit.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace skinny {

namespace {

constexpr int ctz_pow2(int x) { return x <= 1 ? 0 : 1 + ctz_pow2(x >> 1); }
constexpr int next_pow2(int x) { return x <= 1 ? 1 : 2 * next_pow2((x + 1) / 2); }

// columns reduced together: at most gemv_group_max(M), which keeps G*M <= 32
// values per lane; a wave that owns fewer columns reduces them one by one
constexpr int gemv_group_max(int M) { return (32 / next_pow2(M)) < 4 ? (32 / next_pow2(M)) : 4; }

template <int M, int G>
struct GemvShape {
  static_assert(G >= 1 && G <= gemv_group_max(M), "group size");
  static constexpr int P = M * G;
  static constexpr int P2 = next_pow2(P);
  static constexpr int LV = ctz_pow2(P2);  // transposed levels (<= 6)
};

__device__ __forceinline__ float fbits(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t ubits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Device-coherent accesses for data handed from one workgroup to another in
// the same launch.  Relaxed agent-scope atomic stores/loads compile to plain
// global stores/loads with the sc1 (device scope) bit: they are coherent
// across the XCDs' L2 caches without the whole-L2 write-back and invalidate
// that an agent-scope fence costs.  A writer waits for its stores to complete
// (s_waitcnt) before it counts itself in with an atomic; the reader issues its
// loads only after its atomic returned the final count.
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void wait_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // every outstanding load and store of this wave completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return fbits(__builtin_amdgcn_update_dpp(0u, ubits(x), CTRL, 0xF, 0xF, false));
}

// DPP controls: row_mirror (l ^ 15 in a row of 16), row_half_mirror (l ^ 7),
// quad_perm [2,3,0,1] (l ^ 2), quad_perm [1,0,3,2] (l ^ 1)
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppXor1 = 0xB1;

// level L of the fixed tree: partner lane and the lane bit that picks the kept half
template <int L>
struct Level;
template <> struct Level<0> { static constexpr int bit = 3; static constexpr int dpp = kDppRowMirror; };
template <> struct Level<1> { static constexpr int bit = 2; static constexpr int dpp = kDppRowHalfMirror; };
template <> struct Level<2> { static constexpr int bit = 1; static constexpr int dpp = kDppXor2; };
template <> struct Level<3> { static constexpr int bit = 0; static constexpr int dpp = kDppXor1; };
template <> struct Level<4> { static constexpr int bit = 4; static constexpr int dpp = -16; };  // permlane16 swap
template <> struct Level<5> { static constexpr int bit = 5; static constexpr int dpp = -32; };  // permlane32 swap

// One tree level.  CUR live values enter; if the level is transposed (L < LV)
// CUR/2 leave, else CUR == 1 and every lane keeps the full sum.
template <int L, int LV, int CUR, int NV>
__device__ __forceinline__ void tree_level(float (&v)[NV], int lane, int& idx) {
  constexpr int bit = Level<L>::bit;
  constexpr int ctrl = Level<L>::dpp;
  if constexpr (L < LV) {
    constexpr int H = CUR / 2;
    const bool hi = (lane >> bit) & 1;
    if constexpr (ctrl >= 0) {
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float mine = hi ? v[i + H] : v[i];
        const float send = hi ? v[i] : v[i + H];
        v[i] = mine + dpp_mov<ctrl>(send);
      }
    } else {
#pragma unroll
      for (int i = 0; i < H; ++i) {
        // swaps the upper half of the first operand's lane pairs with the
        // lower half of the second's: afterwards the low lanes hold
        // (v[i] of lane, v[i] of partner) and the high lanes
        // (v[i+H] of partner, v[i+H] of lane)
        auto r = (ctrl == -16)
                     ? __builtin_amdgcn_permlane16_swap(ubits(v[i]), ubits(v[i + H]), false, false)
                     : __builtin_amdgcn_permlane32_swap(ubits(v[i]), ubits(v[i + H]), false, false);
        v[i] = fbits(r[0]) + fbits(r[1]);
      }
    }
    if (hi) idx += H;
  } else {
    if constexpr (ctrl >= 0) {
      v[0] = v[0] + dpp_mov<ctrl>(v[0]);
    } else {
      auto r = (ctrl == -16) ? __builtin_amdgcn_permlane16_swap(ubits(v[0]), ubits(v[0]), false, false)
                             : __builtin_amdgcn_permlane32_swap(ubits(v[0]), ubits(v[0]), false, false);
      v[0] = fbits(r[0]) + fbits(r[1]);
    }
  }
}

template <int LV>
constexpr int plain_lane_mask() {
  constexpr int bits[6] = {3, 2, 1, 0, 4, 5};
  int mask = 0;
  for (int L = LV; L < 6; ++L) mask |= 1 << bits[L];
  return mask;
}

// live values entering level L
constexpr int live_at(int L, int LV, int NV) { return L <= LV ? (NV >> L) : 1; }

// Reduce NV = 2^LV values per lane over the 64 lanes.  Afterwards v[0] of a
// lane holds the full sum of value `idx`; the lanes with (lane & mask) == 0
// hold each value exactly once.
template <int LV, int NV>
__device__ __forceinline__ float wave_tree(float (&v)[NV], int lane, int& idx) {
  idx = 0;
  tree_level<0, LV, live_at(0, LV, NV)>(v, lane, idx);
  tree_level<1, LV, live_at(1, LV, NV)>(v, lane, idx);
  tree_level<2, LV, live_at(2, LV, NV)>(v, lane, idx);
  tree_level<3, LV, live_at(3, LV, NV)>(v, lane, idx);
  tree_level<4, LV, live_at(4, LV, NV)>(v, lane, idx);
  tree_level<5, LV, live_at(5, LV, NV)>(v, lane, idx);
  return v[0];
}

// the value stored for a finished sum: the sum itself, or the scalar gate's
// sigmoid of it (an IEEE divide of 1 by 1 + e^-x; the exponential is the
// device library's expf).  EPI is a template argument, so the plain kernels
// carry no trace of the gate.
template <int EPI>
__device__ __forceinline__ float gemv_finish(float sum) {
  if constexpr (EPI == kEpiSigmoid) {
    return 1.0f / (1.0f + expf(-sum));
  } else {
    return sum;
  }
}

template <int WK>
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& w, float acc) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t ap = a[p];
    const uint32_t wp = w[p];
    if constexpr (WK == WK_BF16) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(ap), as_b2(wp), acc, false);
    } else {
      acc = __builtin_amdgcn_fdot2(as_h2(ap), as_h2(wp), acc, false);
    }
  }
  return acc;
}

// Raw weight registers of one (column, chunk): 16 bytes of f16/bf16, or 8
// bytes of codes plus the block's scale for Q8_0.
template <int WK>
struct WChunk {
  u32x4 v;
};
template <>
struct WChunk<WK_Q8> {
  u32x2 codes;
  uint16_t scale;
};

template <int WK>
__device__ __forceinline__ void load_w(WChunk<WK>& dst, const GemvArgs& g, int64_t j, int chunk) {
  if constexpr (WK == WK_Q8) {
    const int8_t* wq = (const int8_t*)g.W;
    dst.codes = *(const u32x2*)(wq + j * g.k + (int64_t)chunk * 8);
    dst.scale = g.scales[j * (g.k >> 5) + (chunk >> 2)];
  } else {
    const uint16_t* w16 = (const uint16_t*)g.W;
    dst.v = *(const u32x4*)(w16 + j * g.k + (int64_t)chunk * 8);
  }
}

template <int WK>
__device__ __forceinline__ void zero_w(WChunk<WK>& dst) {
  if constexpr (WK == WK_Q8) {
    dst.codes = u32x2{0u, 0u};
    dst.scale = 0;
  } else {
    dst.v = u32x4{0u, 0u, 0u, 0u};
  }
}

template <int WK>
__device__ __forceinline__ u32x4 w_as_halves(const WChunk<WK>& w) {
  if constexpr (WK == WK_Q8) {
    return q8_dequant8(w.codes, half_from_bits(w.scale));
  } else {
    return w.v;
  }
}

// Chunk c (eight elements) of A row r as eight 16-bit values: loaded as
// stored, or (AK = kAF32) two 16-byte words of fp32 rounded to bf16 on the
// way in -- the window-row cast fused into the GEMV's A load.
template <int AK>
__device__ __forceinline__ u32x4 load_a8(const GemvArgs& g, int r, int c) {
  if constexpr (AK == kAF32) {
    const u32x4* p = (const u32x4*)((const float*)g.A + (int64_t)r * g.lda + (int64_t)c * 8);
    return bf16x8_rne(p[0], p[1]);
  } else {
    return *(const u32x4*)((const uint16_t*)g.A + (int64_t)r * g.lda + (int64_t)c * 8);
  }
}

// ---------------------------------------------------------------------------
// The GEMV kernel.  M rows (template), T chunk slots per lane, weight kind WK,
// output kind CK, G columns reduced per pass, epilogue EPI, A kind AK.  G changes only how many
// columns share one pass of the reduction tree, never a column's arithmetic.
//
// Wave -> work: with S <= kGemvBlockSplitMax k splits, a workgroup holds
// cg_per_block column ranges and S waves per range (wave w: split w % S,
// range w / S).  Each wave reduces its sums over its 64 lanes, parks them in
// LDS, and after one barrier the block adds the S splits in the fixed order
// s = 0..S-1 and writes C.  With more splits the waves of one range sit in
// different workgroups: each writes its sums to partial[s][r][j], makes them
// visible device-wide and counts itself in on its range; the wave that arrives
// last adds the S partials in the same fixed order.  No wave ever waits for
// another workgroup.  Either way row r sees the same arithmetic at every m.
// The range counters live in the caller's workspace, start at zero and are
// left at zero.
// ---------------------------------------------------------------------------
template <int M, int T, int WK, int CK, int G, int EPI, int AK>
__global__ __launch_bounds__(64 * kGemvMaxWavesPerBlock) void gemv_rows_kernel(GemvArgs g) {
  using Shape = GemvShape<M, G>;
  constexpr int P = Shape::P;
  constexpr int P2 = Shape::P2;
  constexpr int LV = Shape::LV;
  static_assert(LV <= 6, "at most 64 values per lane");

  // sums of one block's waves: [wave][column of the wave][row]
  __shared__ float red[kGemvMaxWavesPerBlock * kGemvCpwMax * M];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wpb = blockDim.x >> 6;
  const bool in_block = g.S <= kGemvBlockSplitMax;
  int s, wc;
  bool active;
  if (in_block) {
    const int cg = wave / g.S;
    s = wave - cg * g.S;
    wc = blockIdx.x * g.cg_per_block + cg;
    active = cg < g.cg_per_block && wc < g.waves_per_split;
  } else {
    const int gw = blockIdx.x * wpb + wave;
    s = gw / g.waves_per_split;
    active = s < g.S;  // trailing waves of the last block have no columns
    wc = active ? gw - s * g.waves_per_split : 0;
  }
  if (!active) wc = 0;
  const int64_t j0 = (int64_t)wc * g.cpw;
  const int ncol = active ? (int)min((int64_t)g.cpw, g.n - j0) : 0;

  // Unsplit k (S = 1) with four or more rows: every wave of the block needs
  // the same A slice (chunks 0 .. 64 T - 1 of every row), so the block loads
  // it once into LDS and each wave reads its chunks from there, instead of
  // every wave fetching all of A through its own load path.
  constexpr bool kStageA = M >= 4;
  __shared__ u32x4 sAr[kStageA ? M * 64 * T : 1];
  const bool stage_a = kStageA && g.S == 1;
  u32x4 a_share[kStageA ? (M * 64 * T + 255) / 256 : 1];
  if (stage_a) {
    // issued before the weight loads, so their latencies overlap
#pragma unroll
    for (int i = 0; i < (kStageA ? (M * 64 * T + 255) / 256 : 0); ++i) {
      const int e = (int)threadIdx.x + i * (int)blockDim.x;
      const int r = e / (64 * T);
      const int c = e - r * (64 * T);
      a_share[i] = (e < M * 64 * T && c < g.nchunks) ? load_a8<AK>(g, r, c) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  int chunk[T];
  bool valid[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    chunk[t] = s * 64 * T + t * 64 + lane;
    valid[t] = active && chunk[t] < g.nchunks;
  }

  // every weight load of the wave, issued before anything else waits
  WChunk<WK> w[kGemvCpwMax][T];
#pragma unroll
  for (int c = 0; c < kGemvCpwMax; ++c) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
      if (c < ncol && valid[t]) {
        load_w<WK>(w[c][t], g, j0 + c, chunk[t]);
      } else {
        zero_w<WK>(w[c][t]);
      }
    }
  }

  // the wave's A slice, kept in registers for all its columns
  u32x4 a[T][M];
  if (stage_a) {
#pragma unroll
    for (int i = 0; i < (kStageA ? (M * 64 * T + 255) / 256 : 0); ++i) {
      const int e = (int)threadIdx.x + i * (int)blockDim.x;
      if (e < M * 64 * T) sAr[e] = a_share[i];
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < M; ++r) a[t][r] = sAr[(r * T + t) * 64 + lane];
  } else {
#pragma unroll
    for (int t = 0; t < T; ++t) {
#pragma unroll
      for (int r = 0; r < M; ++r) {
        a[t][r] = valid[t] ? load_a8<AK>(g, r, chunk[t]) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  if (active) {

    constexpr int plain_mask = plain_lane_mask<LV>();
    const bool writer_lane = (lane & plain_mask) == 0;

#pragma unroll
    for (int c0 = 0; c0 < kGemvCpwMax; c0 += G) {
      if (c0 >= ncol) break;
      float v[P2];
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        u32x4 wh[T];
#pragma unroll
        for (int t = 0; t < T; ++t) wh[t] = w_as_halves<WK>(w[(c0 + gi) < kGemvCpwMax ? (c0 + gi) : 0][t]);
#pragma unroll
        for (int r = 0; r < M; ++r) {
          float acc = 0.0f;
#pragma unroll
          for (int t = 0; t < T; ++t) acc = dot8<WK>(a[t][r], wh[t], acc);
          v[gi * M + r] = acc;
        }
      }
#pragma unroll
      for (int i = P; i < P2; ++i) v[i] = 0.0f;

      int idx;
      const float sum = wave_tree<LV>(v, lane, idx);
      const int gi = idx / M;
      const int r = idx - gi * M;
      if (writer_lane && idx < P && c0 + gi < ncol) {
        const int64_t j = j0 + c0 + gi;
        if (g.S == 1) {
          store_out<CK>(g.C, (int64_t)r * g.ldc + j, gemv_finish<EPI>(sum));
        } else if (in_block) {
          red[(wave * kGemvCpwMax + c0 + gi) * M + r] = sum;
        } else {
          st_dev(g.partial + ((int64_t)s * M + r) * g.n + j, sum);
        }
      }
    }

    if (!in_block) {
      wait_mem();  // this wave's partials have reached the device-coherent level
      uint32_t old = 0;
      if (lane == 0) old = atomicAdd(&g.counters[wc], 1u);
      old = __shfl(old, 0, 64);
      if (old == (uint32_t)(g.S - 1)) {
        // every split of this column range has counted in: add them in order
        for (int e = lane; e < M * ncol; e += 64) {
          const int r = e / ncol;
          const int64_t j = j0 + (e - r * ncol);
          float acc = ld_dev(g.partial + (int64_t)r * g.n + j);
          for (int q = 1; q < g.S; ++q) acc += ld_dev(g.partial + ((int64_t)q * M + r) * g.n + j);
          store_out<CK>(g.C, (int64_t)r * g.ldc + j, gemv_finish<EPI>(acc));
        }
        if (lane == 0) g.counters[wc] = 0u;  // ready for the next call
      }
    }
  }

  if (in_block && g.S > 1) {
    __syncthreads();  // every wave's sums are in LDS
    const int per_range = g.cpw * M;
    for (int e = threadIdx.x; e < g.cg_per_block * per_range; e += blockDim.x) {
      const int cg = e / per_range;
      const int c = (e - cg * per_range) / M;
      const int r = e - cg * per_range - c * M;
      const int64_t j = (int64_t)(blockIdx.x * g.cg_per_block + cg) * g.cpw + c;
      if (j >= g.n) continue;  // past the last column (or the last range)
      const int w0 = cg * g.S;
      float acc = red[(w0 * kGemvCpwMax + c) * M + r];
      for (int q = 1; q < g.S; ++q) acc += red[((w0 + q) * kGemvCpwMax + c) * M + r];
      store_out<CK>(g.C, (int64_t)r * g.ldc + j, gemv_finish<EPI>(acc));
    }
  }
}

// --- kernel table and launcher (instantiated once per weight type) ---------
typedef void (*gemv_fn)(GemvArgs);

// [group: 1 column, gemv_group_max(M) columns][C kind: f32, f16, bf16]
template <int M, int T, int WK, int AK>
struct GemvRow {
  static constexpr int GM = gemv_group_max(M);
  static constexpr gemv_fn out[2][3] = {
      {gemv_rows_kernel<M, T, WK, CK_F32, 1, kEpiNone, AK>, gemv_rows_kernel<M, T, WK, CK_F16, 1, kEpiNone, AK>,
       gemv_rows_kernel<M, T, WK, CK_BF16, 1, kEpiNone, AK>},
      {gemv_rows_kernel<M, T, WK, CK_F32, GM, kEpiNone, AK>, gemv_rows_kernel<M, T, WK, CK_F16, GM, kEpiNone, AK>,
       gemv_rows_kernel<M, T, WK, CK_BF16, GM, kEpiNone, AK>}};
};

// the scalar gate's kernels (sigmoid epilogue; f32 or f16 gate values)
template <int M, int T, int WK, int AK>
struct GemvGateRow {
  static constexpr int GM = gemv_group_max(M);
  static constexpr gemv_fn out[2][3] = {
      {gemv_rows_kernel<M, T, WK, CK_F32, 1, kEpiSigmoid, AK>,
       gemv_rows_kernel<M, T, WK, CK_F16, 1, kEpiSigmoid, AK>, nullptr},
      {gemv_rows_kernel<M, T, WK, CK_F32, GM, kEpiSigmoid, AK>,
       gemv_rows_kernel<M, T, WK, CK_F16, GM, kEpiSigmoid, AK>, nullptr}};
};

template <int T, int WK, int AK, int... Ms>
gemv_fn gemv_pick(int m, int group, int out_kind) {
  const gemv_fn(*tbl[])[3] = {GemvRow<Ms, T, WK, AK>::out...};
  return tbl[m - 1][group][out_kind];
}

template <int T, int WK, int AK, int... Ms>
gemv_fn gemv_pick_gate(int m, int group, int out_kind) {
  const gemv_fn(*tbl[])[3] = {GemvGateRow<Ms, T, WK, AK>::out...};
  return tbl[m - 1][group][out_kind];
}

// AK = kAF32 is instantiated for bf16 weights only (its own translation unit)
template <int WK, int AK = kA16>
hipError_t launch_gemv_kind(const GemvArgs& args, int m, int T, int out_kind, int waves_per_block,
                            hipStream_t stream) {
  static_assert(AK == kA16 || WK == WK_BF16, "fp32 rows feed bf16 weights only");
  if (args.a_kind != AK) return hipErrorInvalidValue;
  if (m < 1 || m > kGemvMaxM || (T != 1 && T != 2) || out_kind < 0 || out_kind > 2 ||
      waves_per_block < 1 || waves_per_block > kGemvMaxWavesPerBlock || args.cpw < 1 ||
      args.cpw > kGemvCpwMax || (args.S == 1 && waves_per_block < 4))
    return hipErrorInvalidValue;  // (unsplit blocks stage A with at least 256 threads)
  // one column per pass when the wave owns fewer columns than a full group
  const int group = args.cpw < gemv_group_max(m) ? 0 : 1;
  gemv_fn fn = nullptr;
  if (args.epilogue == kEpiNone) {
    fn = T == 1 ? gemv_pick<1, WK, AK, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(m, group, out_kind)
                : gemv_pick<2, WK, AK, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(m, group, out_kind);
  } else if constexpr (WK == WK_BF16) {  // the gate: bf16 weights only
    if (args.epilogue == kEpiSigmoid)
      fn = T == 1
               ? gemv_pick_gate<1, WK, AK, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(m, group, out_kind)
               : gemv_pick_gate<2, WK, AK, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 16>(m, group, out_kind);
  }
  if (fn == nullptr) return hipErrorInvalidValue;
  int64_t blocks;
  if (args.S <= kGemvBlockSplitMax) {
    if (args.cg_per_block < 1 || args.cg_per_block * args.S != waves_per_block) return hipErrorInvalidValue;
    blocks = (args.waves_per_split + args.cg_per_block - 1) / args.cg_per_block;
  } else {
    const int64_t waves = (int64_t)args.S * args.waves_per_split;
    blocks = (waves + waves_per_block - 1) / waves_per_block;
  }
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(64 * waves_per_block), 0, stream, args);
  return hipGetLastError();
}

}  // namespace

}  // namespace skinny
