// gemm_inst.hip -- instantiates the MFMA GEMM kernels of one weight kind
// (every tile, output kind and launch shape of gemm_kernel.h) and defines
// its launcher GEMM_LAUNCHER.  The build compiles this file once per weight
// kind with -DGEMM_WK=... -DGEMM_LAUNCHER=..., so the kernels compile in
// parallel.
#include "gemm_kernel.h"

#if !defined(GEMM_WK) || !defined(GEMM_LAUNCHER)
#error "gemm_inst.hip is compiled with GEMM_WK and GEMM_LAUNCHER defined"
#endif

namespace skinny {

hipError_t GEMM_LAUNCHER(int tile_id, const GemmArgs& args, int c_kind, int shape, int64_t blocks, int threads,
                         hipStream_t stream) {
  return launch_gemm_kind<GEMM_WK>(tile_id, args, c_kind, shape, blocks, threads, stream);
}

}  // namespace skinny
