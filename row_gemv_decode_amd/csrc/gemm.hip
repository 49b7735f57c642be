// gemm.hip -- the GEMM tile table, launch dispatch and the ordered k-chunk
// reduce, for gfx950 (MI355X).  The kernels are in gemm_kernel.h, compiled
// per weight kind by gemm_inst.hip.
#include "gemm_kernel.h"

namespace skinny {

// the launchers of gemm_inst.hip, one object per weight kind
hipError_t launch_gemm_f16(int, const GemmArgs&, int, int, int64_t, int, hipStream_t);
hipError_t launch_gemm_bf16(int, const GemmArgs&, int, int, int64_t, int, hipStream_t);
hipError_t launch_gemm_q8(int, const GemmArgs&, int, int, int64_t, int, hipStream_t);
hipError_t launch_gemm_q4(int, const GemmArgs&, int, int, int64_t, int, hipStream_t);
hipError_t launch_gemm_q2(int, const GemmArgs&, int, int, int64_t, int, hipStream_t);

namespace {

// C[r][c] = partial[0][r][c] + partial[1][r][c] + ... in that order.  All of
// an element's partials are loaded before the first add (one memory round
// trip instead of one per chunk); the adds keep the chunk order.
constexpr int kMaxSplits = 16;  // the plan cuts k into at most this many chunks

template <int CK>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs g) {
  const int64_t total = g.M * g.N;
  const int64_t plane = total;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t r = e / g.N;
    const int64_t c = e - r * g.N;
    float part[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) part[s] = s < g.splits ? g.partial[s * plane + e] : 0.0f;
    float acc = part[0];
#pragma unroll
    for (int s = 1; s < kMaxSplits; ++s)
      if (s < g.splits) acc += part[s];
    store_out<CK>(g.C, r * g.ldc + c, acc);
  }
}

#define SKINNY_GEMM_INFO(TM, TN, WM, WN, NS, XT, NAME) GemmTileInfo{TM, TN, WM, WN, NAME},
const GemmTileInfo kTileTable[] = {SKINNY_GEMM_TILE_LIST(SKINNY_GEMM_INFO)};
#undef SKINNY_GEMM_INFO

const GemmTileInfo* tile_infos() { return kTileTable; }

constexpr int kTileCount = (int)(sizeof(kTileTable) / sizeof(kTileTable[0]));

}  // namespace

int gemm_tile_count() { return kTileCount; }

const GemmTileInfo& gemm_tile(int id) { return tile_infos()[id]; }

bool gemm_tile_chunkable(int id) {
  const GemmTileInfo& t = tile_infos()[id];
  return gemm_chunkable(t.tm, t.tn, t.wm, t.wn);
}

hipError_t launch_gemm(int tile_id, const GemmArgs& args, int w_kind, int c_kind, int shape,
                       hipStream_t stream) {
  if (tile_id < 0 || tile_id >= kTileCount || w_kind < WK_F16 || w_kind > WK_Q2 || c_kind < 0 || c_kind > 2 ||
      shape < kGemmPlain || shape > kGemmFold)
    return hipErrorInvalidValue;
  const GemmTileInfo& t = tile_infos()[tile_id];
  const int64_t nk = (args.K + kBK - 1) / kBK;
  if (args.splits < 1 || args.kt_per_split < 1 ||
      (args.splits > 1 && ((int64_t)(args.splits - 1) * args.kt_per_split >= nk ||
                           (int64_t)args.splits * args.kt_per_split < nk || args.partial == nullptr)))
    return hipErrorInvalidValue;
  const int64_t blocks = ((args.M + t.tm - 1) / t.tm) * ((args.N + t.tn - 1) / t.tn) * args.splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  if (shape == kGemmChunked) {
    // a chunked launch folds between pairs of k-tiles: chunks of even length
    if (args.splits != 1 || !gemm_tile_chunkable(tile_id) || (args.kt_per_split % 2 != 0 && args.kt_per_split < nk))
      return hipErrorInvalidValue;
  } else if (shape == kGemmFold) {
    if (args.splits < 2 || !gemm_tile_foldable(tile_id) || args.counters == nullptr) return hipErrorInvalidValue;
  }
  const int threads = 64 * t.wm * t.wn;
  switch (w_kind) {
    case WK_F16: return launch_gemm_f16(tile_id, args, c_kind, shape, blocks, threads, stream);
    case WK_BF16: return launch_gemm_bf16(tile_id, args, c_kind, shape, blocks, threads, stream);
    case WK_Q8: return launch_gemm_q8(tile_id, args, c_kind, shape, blocks, threads, stream);
    case WK_Q4: return launch_gemm_q4(tile_id, args, c_kind, shape, blocks, threads, stream);
    case WK_Q2: return launch_gemm_q2(tile_id, args, c_kind, shape, blocks, threads, stream);
  }
  return hipErrorInvalidValue;
}

bool gemm_tile_foldable(int id) { return gemm_tile_chunkable(id); }

hipError_t launch_splitk_reduce(const GemmArgs& args, int c_kind, hipStream_t stream) {
  if (args.splits < 2 || args.splits > kMaxSplits || args.partial == nullptr || c_kind < 0 || c_kind > 2)
    return hipErrorInvalidValue;
  int64_t blocks = (args.M * args.N + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  const auto fn = c_kind == CK_F32 ? splitk_reduce_kernel<CK_F32>
                : c_kind == CK_F16 ? splitk_reduce_kernel<CK_F16> : splitk_reduce_kernel<CK_BF16>;
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(256), 0, stream, args);
  return hipGetLastError();
}

}  // namespace skinny
