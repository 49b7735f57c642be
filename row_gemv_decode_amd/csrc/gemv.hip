// gemv.hip -- the per-row top-k launch, the standalone block dequants and the
// GEMV launch dispatch, for gfx950 (MI355X).  The GEMV kernel itself is in
// gemv_kernel.h.
#include "gemv_kernel.h"
#include "skinny.h"

namespace skinny {

// the launchers of gemv_inst.hip, one object per (weight kind, A kind, T)
#define SKINNY_GEMV_LAUNCHERS(X) \
  X(launch_gemv_f16_t1) X(launch_gemv_f16_t2) X(launch_gemv_bf16_t1) X(launch_gemv_bf16_t2) \
  X(launch_gemv_q8_t1) X(launch_gemv_q8_t2) X(launch_gemv_q4_t1) X(launch_gemv_q4_t2) \
  X(launch_gemv_q2_t1) X(launch_gemv_q2_t2) X(launch_gemv_bf16_a32_t1) X(launch_gemv_bf16_a32_t2)
#define SKINNY_DECLARE_LAUNCHER(name) hipError_t name(const GemvArgs&, int, int, int, hipStream_t);
SKINNY_GEMV_LAUNCHERS(SKINNY_DECLARE_LAUNCHER)
#undef SKINNY_DECLARE_LAUNCHER

namespace {

// ---------------------------------------------------------------------------
// Per-row top-k, one wavefront per row (Strata PR #109, "What": one multi-row
// top-10 launch over the window's tokens, the row taken from the block index).
// Order: value descending, equal values (IEEE ==, so -0 == +0) by lower column
// first; the result carries the logit's own bits.  Logits are not NaN (a NaN
// logit's rank is unspecified).
//
// Values are compared as order keys: the float's bits with the magnitude bits
// of negative values flipped, read as a signed integer, and -0 mapped to +0's
// key; for non-NaN values the key order is IEEE order and equal keys are
// IEEE-equal values.  Integer keys let each reduction level be one DPP max.
//
// Fast path (n <= 64 * NC): lane l holds columns l, l + 64, ... in NC
// registers, sorted once per lane (a stable odd-even transposition sort, so
// equal values keep increasing columns).  Each round takes the wave maximum of
// the lanes' head keys and a ballot of the lanes whose head equals it: one
// lane in the ballot owns the winner outright, several (a tie) fall back to
// the smallest column among them.  The owner pops its head and lane t keeps
// the t-th winner, so the results leave in one coalesced store.
// Generic path (larger n): each round rescans the row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int order_key(float x) {
  uint32_t b = ubits(x);
  if (b == 0x80000000u) b = 0u;  // -0 ranks with +0
  return (int)(b ^ ((uint32_t)((int)b >> 31) & 0x7fffffffu));
}

template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int x) {
  return (int)__builtin_amdgcn_update_dpp(0u, (uint32_t)x, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, dpp_mov_i<kDppXor1>(v));
  v = max(v, dpp_mov_i<kDppXor2>(v));
  v = max(v, dpp_mov_i<kDppRowHalfMirror>(v));
  v = max(v, dpp_mov_i<kDppRowMirror>(v));
  auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)r16[0], (int)r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  v = max((int)r32[0], (int)r32[1]);
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, dpp_mov_i<kDppXor1>(v));
  v = min(v, dpp_mov_i<kDppXor2>(v));
  v = min(v, dpp_mov_i<kDppRowHalfMirror>(v));
  v = min(v, dpp_mov_i<kDppRowMirror>(v));
  auto r16 = __builtin_amdgcn_permlane16_swap((uint32_t)v, (uint32_t)v, false, false);
  v = min((int)r16[0], (int)r16[1]);
  auto r32 = __builtin_amdgcn_permlane32_swap((uint32_t)v, (uint32_t)v, false, false);
  v = min((int)r32[0], (int)r32[1]);
  return v;
}

// (key, j) comes after (pkey, pj) in the order above
__device__ __forceinline__ bool after(int key, int j, int pkey, int pj) {
  return key < pkey || (key == pkey && j > pj);
}

constexpr int kNoColumn = 0x7fffffff;
constexpr int kNoKey = (int)0x80000000;  // below every non-NaN value's key

// the float whose order key is `key` (-0 comes back as +0)
__device__ __forceinline__ float key_value(int key) {
  return fbits((uint32_t)key ^ ((uint32_t)(key >> 31) & 0x7fffffffu));
}

// TK > 0: topk is TK, known at compile time (the fast pass unrolls); 0: runtime
template <int NC, int TK>
__device__ __forceinline__ void wave_topk_row_regs(const float* row, int n, int topk_arg, int32_t* out_idx,
                                                   float* out_val, int lane) {
  int key[NC];
  int jj[NC];
  float x[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {  // every load in flight before the first key
    const int j = lane + 64 * u;
    x[u] = j < n ? row[j] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int j = lane + 64 * u;
    const bool ok = j < n;
    key[u] = ok ? order_key(x[u]) : kNoKey;
    jj[u] = ok ? j : kNoColumn;
  }
  // stable sort of the lane's slots into rank order: the slots start in
  // increasing column order and only a strictly larger key moves up, so equal
  // keys keep increasing columns without comparing them
#pragma unroll
  for (int round = 0; round < NC; ++round) {
#pragma unroll
    for (int u = round & 1; u + 1 < NC; u += 2) {
      const bool swap = key[u] < key[u + 1];
      const int tk = key[u];
      const int tj = jj[u];
      key[u] = swap ? key[u + 1] : key[u];
      jj[u] = swap ? jj[u + 1] : jj[u];
      key[u + 1] = swap ? tk : key[u + 1];
      jj[u + 1] = swap ? tj : jj[u + 1];
    }
  }
  // Each round: the winner is the lane whose head holds the wave maximum (a
  // tie takes the lowest column among the tied heads); it pops its head and
  // notes the round in a bit mask.  A lane pops in order, so its k-th win is
  // its k-th sorted slot: after the last round every lane writes its wins to
  // LDS by round, and lane t reads round t.  No lane index crosses to the
  // scalar unit inside the loop: a round is the maximum's reduction plus a
  // few selects.
  int skey[NC];
  int sjj[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    skey[u] = key[u];
    sjj[u] = jj[u];
  }
  // the winner pops its head: each slot takes the next one under an all-ones
  // mask (one bit-field insert per slot)
  auto pop = [&](bool mine) __attribute__((always_inline)) {
    const uint32_t pm = 0u - (uint32_t)mine;
#pragma unroll
    for (int u = 0; u + 1 < NC; ++u) {
      key[u] = (int)((pm & (uint32_t)key[u + 1]) | (~pm & (uint32_t)key[u]));
      jj[u] = (int)((pm & (uint32_t)jj[u + 1]) | (~pm & (uint32_t)jj[u]));
    }
    key[NC - 1] = (int)((pm & (uint32_t)kNoKey) | (~pm & (uint32_t)key[NC - 1]));
    jj[NC - 1] = (int)((pm & (uint32_t)kNoColumn) | (~pm & (uint32_t)jj[NC - 1]));
  };
  // Fast pass: every lane whose head equals the maximum pops, and the
  // ballots only record whether any round had two such lanes (a tie), off
  // the rounds' critical path.  A tie makes the pass wrong from that round
  // on, so then the rounds are redone from the sorted slots with the tie
  // rule (the lowest column among the tied heads wins).
  const int topk = TK > 0 ? TK : topk_arg;
  uint32_t rounds_won = 0;
  uint64_t ties = 0;
  auto fast_round = [&](int t) __attribute__((always_inline)) {
    const int kmax = wave_max_i32(key[0]);  // the same in every lane
    const bool mine = key[0] == kmax;
    const uint64_t b = __builtin_amdgcn_ballot_w64(mine);
    ties |= b & (b - 1);  // non-zero when two or more lanes hold the maximum
    rounds_won |= (0u - (uint32_t)mine) & (1u << t);
    pop(mine);
  };
  if constexpr (TK > 0) {
#pragma unroll
    for (int t = 0; t < TK; ++t) fast_round(t);
  } else {
    for (int t = 0; t < topk; ++t) fast_round(t);
  }
  if (ties != 0) {  // uniform; equal logits among the leaders, rare
#pragma unroll
    for (int u = 0; u < NC; ++u) {
      key[u] = skey[u];
      jj[u] = sjj[u];
    }
    rounds_won = 0;
    for (int t = 0; t < topk; ++t) {
      const int kmax = wave_max_i32(key[0]);
      bool mine = key[0] == kmax;
      if (__builtin_popcountll(__builtin_amdgcn_ballot_w64(mine)) != 1) {  // uniform
        const int wj = wave_min_i32(mine ? jj[0] : kNoColumn);
        mine = mine && jj[0] == wj;
      }
      rounds_won |= (0u - (uint32_t)mine) & (1u << t);
      pop(mine);
    }
  }
  __shared__ int won_j[SKINNY_TOPK_MAX];
  __shared__ int won_k[SKINNY_TOPK_MAX];
  uint32_t left = rounds_won;
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    if (left != 0) {
      const int r = __builtin_ctz(left);
      won_j[r] = sjj[u];
      won_k[r] = skey[u];
      left &= left - 1;
    }
  }
  __syncthreads();  // one wave: orders the writes before the reads
  if (lane < topk) {
    const int res_j = won_j[lane];
    const int res_k = won_k[lane];
    out_idx[lane] = res_j;
    // the key gives the value's bits back, except that a zero may be -0
    out_val[lane] = res_k == 0 ? row[res_j] : key_value(res_k);
  }
}

__device__ void wave_topk_row_generic(const float* row, int n, int topk, int32_t* out_idx, float* out_val,
                                      int lane) {
  int prev_k = 0;
  int prev_j = -1;
  for (int t = 0; t < topk; ++t) {
    int best = kNoKey;
    for (int j = lane; j < n; j += 64) {
      const int kx = order_key(row[j]);
      if (prev_j < 0 || after(kx, j, prev_k, prev_j)) best = max(best, kx);
    }
    const int kmax = wave_max_i32(best);
    int cand = kNoColumn;
    float cand_v = 0.0f;
    for (int j = lane; j < n; j += 64) {
      const float x = row[j];
      const int kx = order_key(x);
      if (kx == kmax && (prev_j < 0 || after(kx, j, prev_k, prev_j)) && j < cand) {
        cand = j;
        cand_v = x;
      }
    }
    const int wj = wave_min_i32(cand);
    if (cand == wj) {
      out_idx[t] = wj;
      out_val[t] = cand_v;
    }
    prev_k = kmax;
    prev_j = wj;
  }
}

// --- top-k launch: one wavefront per row, blockIdx.x = row -------------------
// NC > 0: rows of at most 64 * NC columns held in registers; NC == 0: generic
template <int NC, int TK>
__global__ __launch_bounds__(64) void topk_rows_kernel(const float* __restrict__ logits, int64_t n,
                                                       int64_t ldl, int32_t* __restrict__ out_idx,
                                                       float* __restrict__ out_val, int topk) {
  const int r = blockIdx.x;
  const float* row = logits + (int64_t)r * ldl;
  int32_t* oi = out_idx + (int64_t)r * topk;
  float* ov = out_val + (int64_t)r * topk;
  if constexpr (NC > 0) {
    wave_topk_row_regs<NC, TK>(row, (int)n, topk, oi, ov, threadIdx.x);
  } else {
    wave_topk_row_generic(row, (int)n, topk, oi, ov, threadIdx.x);
  }
}

// --- window-row cast: fp32 -> bf16, round to nearest even --------------------
// Eight values per thread and step: two 16-byte loads, one 16-byte store; the
// count % 8 tail is converted one value per thread by the first workgroup.
// The conversion is the compiler's float -> __bf16, the same one the bf16
// output path of every kernel uses.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void cast_f32_bf16_kernel(const float* __restrict__ in,
                                                            uint16_t* __restrict__ out, int64_t count) {
  const int64_t groups = count >> 3;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < groups; e += (int64_t)gridDim.x * 256) {
    const f32x4 lo = *(const f32x4*)(in + e * 8);
    const f32x4 hi = *(const f32x4*)(in + e * 8 + 4);
    b8_t v;
    v[0] = (__bf16)lo[0];
    v[1] = (__bf16)lo[1];
    v[2] = (__bf16)lo[2];
    v[3] = (__bf16)lo[3];
    v[4] = (__bf16)hi[0];
    v[5] = (__bf16)hi[1];
    v[6] = (__bf16)hi[2];
    v[7] = (__bf16)hi[3];
    *(u32x4*)(out + e * 8) = __builtin_bit_cast(u32x4, v);
  }
  const int64_t tail = count - (groups << 3);
  if (blockIdx.x == 0 && (int64_t)threadIdx.x < tail) {
    const int64_t i = (groups << 3) + threadIdx.x;
    ((__bf16*)out)[i] = (__bf16)in[i];
  }
}

// --- standalone dequant ----------------------------------------------------
__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const int8_t* __restrict__ qs,
                                                           const uint16_t* __restrict__ d,
                                                           uint16_t* __restrict__ out, int64_t n,
                                                           int64_t k) {
  const int64_t chunks_per_row = k >> 3;
  const int64_t total = n * chunks_per_row;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t j = e / chunks_per_row;
    const int64_t c = e - j * chunks_per_row;
    const u32x2 codes = *(const u32x2*)(qs + j * k + c * 8);
    const _Float16 scale = half_from_bits(d[j * (k >> 5) + (c >> 2)]);
    *(u32x4*)(out + j * k + c * 8) = q8_dequant8(codes, scale);
  }
}

// eight weights per thread and step: four bytes of packed codes
__global__ __launch_bounds__(256) void dequant_q4_0_kernel(const uint8_t* __restrict__ qs,
                                                           const uint16_t* __restrict__ d,
                                                           uint16_t* __restrict__ out, int64_t n,
                                                           int64_t k) {
  const int64_t chunks_per_row = k >> 3;
  const int64_t total = n * chunks_per_row;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t j = e / chunks_per_row;
    const int64_t c = e - j * chunks_per_row;
    const uint32_t codes = *(const uint32_t*)(qs + j * (k >> 1) + c * 4);
    const _Float16 scale = half_from_bits(d[j * (k >> 5) + (c >> 2)]);
    *(u32x4*)(out + j * k + c * 8) = q4_dequant8(codes, scale);
  }
}

// eight weights per thread and step: two bytes of packed codes
__global__ __launch_bounds__(256) void dequant_q2_0_kernel(const uint8_t* __restrict__ qs,
                                                           const uint16_t* __restrict__ d,
                                                           uint16_t* __restrict__ out, int64_t n,
                                                           int64_t k) {
  const int64_t chunks_per_row = k >> 3;
  const int64_t total = n * chunks_per_row;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t j = e / chunks_per_row;
    const int64_t c = e - j * chunks_per_row;
    const uint32_t codes = *(const uint16_t*)(qs + j * (k >> 2) + c * 2);
    const _Float16 scale = half_from_bits(d[j * (k >> 5) + (c >> 2)]);
    *(u32x4*)(out + j * k + c * 8) = q2_dequant8(codes, scale);
  }
}

}  // namespace

hipError_t launch_gemv(const GemvArgs& args, int m, int T, int w_kind, int out_kind,
                       int waves_per_block, hipStream_t stream) {
  if (T != 1 && T != 2) return hipErrorInvalidValue;
  const bool t1 = T == 1;
  if (args.a_kind == kAF32) {
    if (w_kind != WK_BF16) return hipErrorInvalidValue;
    return t1 ? launch_gemv_bf16_a32_t1(args, m, out_kind, waves_per_block, stream)
              : launch_gemv_bf16_a32_t2(args, m, out_kind, waves_per_block, stream);
  }
  switch (w_kind) {
    case WK_F16:
      return t1 ? launch_gemv_f16_t1(args, m, out_kind, waves_per_block, stream)
                : launch_gemv_f16_t2(args, m, out_kind, waves_per_block, stream);
    case WK_BF16:
      return t1 ? launch_gemv_bf16_t1(args, m, out_kind, waves_per_block, stream)
                : launch_gemv_bf16_t2(args, m, out_kind, waves_per_block, stream);
    case WK_Q8:
      return t1 ? launch_gemv_q8_t1(args, m, out_kind, waves_per_block, stream)
                : launch_gemv_q8_t2(args, m, out_kind, waves_per_block, stream);
    case WK_Q4:
      return t1 ? launch_gemv_q4_t1(args, m, out_kind, waves_per_block, stream)
                : launch_gemv_q4_t2(args, m, out_kind, waves_per_block, stream);
    case WK_Q2:
      return t1 ? launch_gemv_q2_t1(args, m, out_kind, waves_per_block, stream)
                : launch_gemv_q2_t2(args, m, out_kind, waves_per_block, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const float* logits, int m, int64_t n, int64_t ldl, int32_t* idx, float* val,
                       int topk, hipStream_t stream) {
  if (topk < 1 || topk > SKINNY_TOPK_MAX || topk > n) return hipErrorInvalidValue;  // the kernels' bounds
  typedef void (*topk_fn)(const float*, int64_t, int64_t, int32_t*, float*, int);
  // top-10 (the router's) gets its own unrolled kernels
  const bool ten = topk == 10;
  const topk_fn fn = n <= 64    ? (ten ? topk_rows_kernel<1, 10> : topk_rows_kernel<1, 0>)
                     : n <= 128 ? (ten ? topk_rows_kernel<2, 10> : topk_rows_kernel<2, 0>)
                     : n <= 256 ? (ten ? topk_rows_kernel<4, 10> : topk_rows_kernel<4, 0>)
                     : n <= 512 ? (ten ? topk_rows_kernel<8, 10> : topk_rows_kernel<8, 0>)
                     : n <= 1024 ? (ten ? topk_rows_kernel<16, 10> : topk_rows_kernel<16, 0>)
                                 : topk_rows_kernel<0, 0>;
  hipLaunchKernelGGL(fn, dim3((unsigned)m), dim3(64), 0, stream, logits, n, ldl, idx, val, topk);
  return hipGetLastError();
}

hipError_t launch_cast_f32_bf16(int64_t count, const float* in, uint16_t* out, hipStream_t stream) {
  const int64_t groups = count >> 3;
  int64_t blocks = (groups + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(cast_f32_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, count);
  return hipGetLastError();
}

hipError_t launch_dequant_q4_0(int64_t n, int64_t k, const uint8_t* qs, const uint16_t* d,
                               uint16_t* out, hipStream_t stream) {
  const int64_t total = n * (k >> 3);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dequant_q4_0_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, qs, d, out,
                     n, k);
  return hipGetLastError();
}

hipError_t launch_dequant_q2_0(int64_t n, int64_t k, const uint8_t* qs, const uint16_t* d,
                               uint16_t* out, hipStream_t stream) {
  const int64_t total = n * (k >> 3);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dequant_q2_0_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, qs, d, out,
                     n, k);
  return hipGetLastError();
}

hipError_t launch_dequant_q8_0(int64_t n, int64_t k, const int8_t* qs, const uint16_t* d,
                               uint16_t* out, hipStream_t stream) {
  const int64_t total = n * (k >> 3);
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(dequant_q8_0_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, qs, d, out,
                     n, k);
  return hipGetLastError();
}

}  // namespace skinny
