// gemv.hip -- the per-row top-k launch, the standalone Q8_0 dequant and the
// GEMV launch dispatch, for gfx950 (MI355X).  The GEMV kernel itself is in
// gemv_kernel.h.
#include "gemv_kernel.h"

namespace skinny {

// one translation unit per weight type (gemv_f16.hip, gemv_bf16.hip, gemv_q8.hip)
hipError_t launch_gemv_f16(const GemvArgs&, int, int, int, int, hipStream_t);
hipError_t launch_gemv_bf16(const GemvArgs&, int, int, int, int, hipStream_t);
hipError_t launch_gemv_q8(const GemvArgs&, int, int, int, int, hipStream_t);

namespace {

// ---------------------------------------------------------------------------
// Per-row top-k, one wavefront per row (Strata PR #109, "What": one multi-row
// top-10 launch over the window's tokens, the row taken from the block index).
// Order: value descending, equal values (IEEE ==, so -0 == +0) by lower column
// first; the result carries the logit's own bits.
//
// Fast path (n <= 64 * NC): lane l holds columns l, l + 64, ... in NC
// registers, sorted once per lane (a stable odd-even transposition sort, so
// equal values keep increasing columns).  Each round takes the wave maximum of
// the lanes' heads (DPP / permlane max) and a ballot of the lanes whose head
// equals it: one lane in the ballot owns the winner outright, several (a tie)
// fall back to the smallest column among them.  The owner pops its head and
// lane t keeps the t-th winner, so the results leave in one coalesced store.
// Generic path (larger n): each round rescans the row.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_mov<kDppXor1>(v));
  v = fmaxf(v, dpp_mov<kDppXor2>(v));
  v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
  auto r16 = __builtin_amdgcn_permlane16_swap(ubits(v), ubits(v), false, false);
  v = fmaxf(fbits(r16[0]), fbits(r16[1]));
  auto r32 = __builtin_amdgcn_permlane32_swap(ubits(v), ubits(v), false, false);
  v = fmaxf(fbits(r32[0]), fbits(r32[1]));
  return v;
}

template <int CTRL>
__device__ __forceinline__ int dpp_mov_i(int x) {
  return (int)__builtin_amdgcn_update_dpp(0u, (uint32_t)x, CTRL, 0xF, 0xF, false);
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

// (v, j) comes after (pv, pj) in the order above
__device__ __forceinline__ bool after(float v, int j, float pv, int pj) {
  return v < pv || (v == pv && j > pj);
}

constexpr int kNoColumn = 0x7fffffff;

template <int NC>
__device__ __forceinline__ void wave_topk_row_regs(const float* row, int n, int topk, int32_t* out_idx,
                                                   float* out_val, int lane) {
  float v[NC];
  int jj[NC];
#pragma unroll
  for (int u = 0; u < NC; ++u) {
    const int j = lane + 64 * u;
    const bool ok = j < n;
    v[u] = ok ? row[j] : -__builtin_inff();
    jj[u] = ok ? j : kNoColumn;
  }
  // stable sort of the lane's slots into rank order
#pragma unroll
  for (int round = 0; round < NC; ++round) {
#pragma unroll
    for (int u = round & 1; u + 1 < NC; u += 2) {
      const bool swap = after(v[u], jj[u], v[u + 1], jj[u + 1]);
      const float tv = v[u];
      const int tj = jj[u];
      v[u] = swap ? v[u + 1] : v[u];
      jj[u] = swap ? jj[u + 1] : jj[u];
      v[u + 1] = swap ? tv : v[u + 1];
      jj[u + 1] = swap ? tj : jj[u + 1];
    }
  }
  int res_j = 0;
  float res_v = 0.0f;
  for (int t = 0; t < topk; ++t) {
    const float wmax = wave_max_f32(v[0]);
    uint64_t ball = __builtin_amdgcn_ballot_w64(v[0] == wmax);
    if (__builtin_popcountll(ball) != 1) {  // wave-uniform; a tie, rare with continuous data
      const int wj = wave_min_i32(((ball >> lane) & 1) ? jj[0] : kNoColumn);
      ball = __builtin_amdgcn_ballot_w64(jj[0] == wj);
    }
    const int owner = ball != 0 ? __builtin_ctzll(ball) : 0;
    const int wj = __builtin_amdgcn_readlane(jj[0], owner);
    const float wv = fbits((uint32_t)__builtin_amdgcn_readlane((int)ubits(v[0]), owner));
    res_j = lane == t ? wj : res_j;
    res_v = lane == t ? wv : res_v;
    const bool mine = lane == owner;
#pragma unroll
    for (int u = 0; u + 1 < NC; ++u) {
      v[u] = mine ? v[u + 1] : v[u];
      jj[u] = mine ? jj[u + 1] : jj[u];
    }
    v[NC - 1] = mine ? -__builtin_inff() : v[NC - 1];
    jj[NC - 1] = mine ? kNoColumn : jj[NC - 1];
  }
  if (lane < topk) {
    out_idx[lane] = res_j;
    out_val[lane] = res_v;
  }
}

__device__ __noinline__ void wave_topk_row_generic(const float* row, int n, int topk, int32_t* out_idx,
                                                   float* out_val, int lane) {
  float prev_v = 0.0f;
  int prev_j = -1;
  for (int t = 0; t < topk; ++t) {
    float best = -__builtin_inff();
    for (int j = lane; j < n; j += 64) {
      const float x = row[j];
      if (prev_j < 0 || after(x, j, prev_v, prev_j)) best = fmaxf(best, x);
    }
    const float wmax = wave_max_f32(best);
    int cand = kNoColumn;
    float cand_v = 0.0f;
    for (int j = lane; j < n; j += 64) {
      const float x = row[j];
      if (x == wmax && (prev_j < 0 || after(x, j, prev_v, prev_j)) && j < cand) {
        cand = j;
        cand_v = x;
      }
    }
    const int wj = wave_min_i32(cand);
    if (cand == wj) {
      out_idx[t] = wj;
      out_val[t] = cand_v;
    }
    prev_v = wmax;
    prev_j = wj;
  }
}

__device__ __forceinline__ void wave_topk_row(const float* row, int n, int topk, int32_t* out_idx,
                                              float* out_val, int lane) {
  if (n <= 64) {
    wave_topk_row_regs<1>(row, n, topk, out_idx, out_val, lane);
  } else if (n <= 128) {
    wave_topk_row_regs<2>(row, n, topk, out_idx, out_val, lane);
  } else if (n <= 256) {
    wave_topk_row_regs<4>(row, n, topk, out_idx, out_val, lane);
  } else if (n <= 512) {
    wave_topk_row_regs<8>(row, n, topk, out_idx, out_val, lane);
  } else if (n <= 1024) {
    wave_topk_row_regs<16>(row, n, topk, out_idx, out_val, lane);
  } else {
    wave_topk_row_generic(row, n, topk, out_idx, out_val, lane);
  }
}

// --- top-k launch: one wavefront per row, blockIdx.x = row -------------------
__global__ __launch_bounds__(64) void topk_rows_kernel(const float* __restrict__ logits, int64_t n,
                                                       int64_t ldl, int32_t* __restrict__ out_idx,
                                                       float* __restrict__ out_val, int topk) {
  const int r = blockIdx.x;
  wave_topk_row(logits + (int64_t)r * ldl, (int)n, topk, out_idx + (int64_t)r * topk,
                out_val + (int64_t)r * topk, threadIdx.x);
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

}  // namespace

hipError_t launch_gemv(const GemvArgs& args, int m, int T, int w_kind, int out_kind,
                       int waves_per_block, hipStream_t stream) {
  switch (w_kind) {
    case WK_F16: return launch_gemv_f16(args, m, T, out_kind, waves_per_block, stream);
    case WK_BF16: return launch_gemv_bf16(args, m, T, out_kind, waves_per_block, stream);
    case WK_Q8: return launch_gemv_q8(args, m, T, out_kind, waves_per_block, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_topk(const float* logits, int m, int64_t n, int64_t ldl, int32_t* idx, float* val,
                       int topk, hipStream_t stream) {
  hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)m), dim3(64), 0, stream, logits, n, ldl, idx, val,
                     topk);
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
