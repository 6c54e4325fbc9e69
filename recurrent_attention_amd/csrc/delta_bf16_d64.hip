// delta_bf16_d64.hip -- delta-rule kernels for d_k = d_v = 64, bf16 inputs.
#include "delta_kernel.h"

namespace la {
LA_DEFINE_DELTA_LAUNCHER(launch_delta_bf16_d64, 64, true)
}  // namespace la
