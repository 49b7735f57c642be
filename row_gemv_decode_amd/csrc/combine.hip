// combine.hip -- the multi-row MoE combine for gfx950 (MI355X).
//
// Strata PR #109, "What": the window's MoE combine is one launch over all of
// its tokens, the token taken from blockIdx.y.  Each token's output row is its
// routed experts' output rows weighted by its routing weights, plus the shared
// expert's row times the shared expert's scalar gate:
//
//   out[t][c] = sum over i < topk of w[t][i] * y[t][i][c]  (+ g[t] * s[t][c])
//
// The routing weights come in as an input (the page does not say how they are
// formed).  One wave per workgroup covers 64 * CPL columns of one token, CPL
// per lane with one 16-byte load per expert row (CPL = 4 fp32 or 8 bf16
// values; every row and the shared row in flight together, so the combine
// costs one memory round trip); the sum is
// a chain of fp32 fused multiply-adds in the order i = 0 .. topk - 1, then the
// shared term, rounded once to the output type.  Nothing depends on m, so a token's row is
// the same bits at every m.  HBM-bound: each input byte is read once.
#include <utility>

#include "device_common.h"

namespace skinny {

namespace {

// columns per lane: one 16-byte load per row.  Measured on MI355X (top-10,
// d = 5120, fp32 rows, graph replay): eight fp32 columns per lane (two loads
// per row) took 2.51 / 2.66 / 2.69 / 2.98 / 3.36 us at m = 1 / 2 / 4 / 8 / 16,
// four 2.44 / 2.51 / 2.53 / 2.87 / 3.22, two (8-byte loads) the same as four
// within 2 %
template <int YK>
constexpr int combine_cpl() { return YK == CK_F32 ? 4 : 8; }

// CPL consecutive values of a row as fp32, one 16-byte load
template <int YK>
__device__ __forceinline__ void load_cols(const void* base, int64_t idx, float (&v)[combine_cpl<YK>()]) {
  if constexpr (YK == CK_F32) {
    const u32x4 q = *(const u32x4*)((const float*)base + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = f32_from_bits(q[e]);
  } else {
    const u32x4 q = *(const u32x4*)((const uint16_t*)base + idx);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = f32_from_bits(q[e] << 16);
      v[2 * e + 1] = f32_from_bits(q[e] & 0xffff0000u);
    }
  }
}

// TK expert rows per token (a template argument, so the loops unroll with no
// per-row branch and every row's load is in flight before the first add)
template <int YK, int OK, int TK>
__global__ __launch_bounds__(64) void moe_combine_kernel(CombineArgs a) {
  constexpr int CPL = combine_cpl<YK>();
  const int64_t c0 = ((int64_t)blockIdx.x * 64 + threadIdx.x) * CPL;
  if (c0 >= a.d) return;  // d % 8 == 0: a lane's columns are all in or all out
  const bool shared = a.shared != nullptr;
  for (int64_t t = blockIdx.y; t < a.m; t += gridDim.y) {
    float v[TK][CPL];
#pragma unroll
    for (int i = 0; i < TK; ++i) load_cols<YK>(a.rows, (t * TK + i) * a.d + c0, v[i]);
    float s[CPL];
    if (shared) load_cols<YK>(a.shared, t * a.d + c0, s);
    const float* w = a.weights + t * TK;
    float acc[CPL];
#pragma unroll
    for (int e = 0; e < CPL; ++e) acc[e] = 0.0f;
#pragma unroll
    for (int i = 0; i < TK; ++i) {
      const float wi = w[i];
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[e] = __builtin_fmaf(wi, v[i][e], acc[e]);
    }
    if (shared) {
      const float g = a.gate[t];
#pragma unroll
      for (int e = 0; e < CPL; ++e) acc[e] = __builtin_fmaf(g, s[e], acc[e]);
    }
    if constexpr (OK == CK_F32) {
      u32x4* o = (u32x4*)((float*)a.out + t * a.d + c0);
#pragma unroll
      for (int q = 0; q < CPL / 4; ++q)
        o[q] = u32x4{__builtin_bit_cast(uint32_t, acc[4 * q]), __builtin_bit_cast(uint32_t, acc[4 * q + 1]),
                     __builtin_bit_cast(uint32_t, acc[4 * q + 2]), __builtin_bit_cast(uint32_t, acc[4 * q + 3])};
    } else if constexpr (CPL == 8) {
      b8_t r;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = (__bf16)acc[e];  // round to nearest even
      *(u32x4*)((uint16_t*)a.out + t * a.d + c0) = __builtin_bit_cast(u32x4, r);
    } else {
      const b2_t lo = {(__bf16)acc[0], (__bf16)acc[1]};  // round to nearest even
      const b2_t hi = {(__bf16)acc[2], (__bf16)acc[3]};
      *(u32x2*)((uint16_t*)a.out + t * a.d + c0) =
          u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
  }
}

typedef void (*combine_fn)(CombineArgs);

// [row kind][out kind] for TK = 1 .. 32
template <int... TKs>
combine_fn combine_pick(int rows_kind, int out_kind, int topk, std::integer_sequence<int, TKs...>) {
  static const combine_fn tbl[2][2][sizeof...(TKs)] = {
      {{moe_combine_kernel<CK_F32, CK_F32, TKs + 1>...}, {moe_combine_kernel<CK_F32, CK_BF16, TKs + 1>...}},
      {{moe_combine_kernel<CK_BF16, CK_F32, TKs + 1>...}, {moe_combine_kernel<CK_BF16, CK_BF16, TKs + 1>...}}};
  return tbl[rows_kind == CK_F32 ? 0 : 1][out_kind == CK_F32 ? 0 : 1][topk - 1];
}

}  // namespace

hipError_t launch_moe_combine(const CombineArgs& args, int rows_kind, int out_kind, hipStream_t stream) {
  if ((rows_kind != CK_F32 && rows_kind != CK_BF16) || (out_kind != CK_F32 && out_kind != CK_BF16) ||
      args.m < 1 || args.d < 8 || args.d % 8 != 0 || args.topk < 1 || args.topk > kCombineMaxTopk)
    return hipErrorInvalidValue;
  const combine_fn fn =
      combine_pick(rows_kind, out_kind, (int)args.topk, std::make_integer_sequence<int, kCombineMaxTopk>{});
  const int64_t cols = 64 * (rows_kind == CK_F32 ? combine_cpl<CK_F32>() : combine_cpl<CK_BF16>());
  const int64_t xb = (args.d + cols - 1) / cols;  // columns per workgroup
  const int64_t yb = args.m < 65535 ? args.m : 65535;  // more tokens: each workgroup takes every 65535th
  if (xb > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(fn, dim3((unsigned)xb, (unsigned)yb), dim3(64), 0, stream, args);
  return hipGetLastError();
}

}  // namespace skinny
