// gemv_f16.hip -- the multi-row GEMV kernels for f16 weights (one
// translation unit per weight type so the instantiations build in parallel).
#include "gemv_kernel.h"

namespace skinny {

hipError_t launch_gemv_f16(const GemvArgs& args, int m, int T, int out_kind, int waves_per_block,
                   hipStream_t stream) {
  return launch_gemv_kind<WK_F16>(args, m, T, out_kind, waves_per_block, stream);
}

}  // namespace skinny
