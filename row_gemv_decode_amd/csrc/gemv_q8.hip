// gemv_q8.hip -- the multi-row GEMV kernels for Q8_0-style weights (one
// translation unit per weight type so the instantiations build in parallel).
#include "gemv_kernel.h"

namespace skinny {

hipError_t launch_gemv_q8(const GemvArgs& args, int m, int T, int out_kind, int waves_per_block,
                   hipStream_t stream) {
  return launch_gemv_kind<WK_Q8>(args, m, T, out_kind, waves_per_block, stream);
}

}  // namespace skinny
