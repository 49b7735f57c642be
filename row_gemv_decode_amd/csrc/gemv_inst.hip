// gemv_inst.hip -- instantiates the multi-row GEMV kernels of one weight
// kind, A kind and chunk count T (gemv_kernel.h), defining the launcher
// GEMV_LAUNCHER.  The build compiles this file once per combination with
// -DGEMV_WK=... -DGEMV_AK=... -DGEMV_T=... -DGEMV_LAUNCHER=..., so the many
// instantiations (rows x columns per wave x output kind x split class)
// compile in parallel.  fp32 A rows (GEMV_AK = kAF32) feed bf16 weights
// only: the window rows' bf16 cast fused into the GEMV's A load.
#include "gemv_kernel.h"

#if !defined(GEMV_WK) || !defined(GEMV_AK) || !defined(GEMV_T) || !defined(GEMV_LAUNCHER)
#error "gemv_inst.hip is compiled with GEMV_WK, GEMV_AK, GEMV_T and GEMV_LAUNCHER defined"
#endif

namespace skinny {

hipError_t GEMV_LAUNCHER(const GemvArgs& args, int m, int out_kind, int waves_per_block, hipStream_t stream) {
  return launch_gemv_kind<GEMV_WK, GEMV_AK, GEMV_T>(args, m, out_kind, waves_per_block, stream);
}

}  // namespace skinny
