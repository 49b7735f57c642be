// gemv_bf16_a32.hip -- the multi-row GEMV kernels for bf16 weights fed by
// fp32 rows of A, each value rounded to bf16 (nearest even) as it is loaded:
// the window rows' bf16 cast fused into the GEMV (its own translation unit so
// the instantiations build in parallel with the others).
#include "gemv_kernel.h"

namespace skinny {

hipError_t launch_gemv_bf16_a32(const GemvArgs& args, int m, int T, int out_kind, int waves_per_block,
                                hipStream_t stream) {
  return launch_gemv_kind<WK_BF16, kAF32>(args, m, T, out_kind, waves_per_block, stream);
}

}  // namespace skinny
