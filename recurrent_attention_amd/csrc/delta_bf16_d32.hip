// delta_bf16_d32.hip -- delta-rule kernels for d_k = d_v = 32, bf16 inputs.
#include "delta_kernel.h"

namespace la {
LA_DEFINE_DELTA_LAUNCHER(launch_delta_bf16_d32, 32, true)
}  // namespace la
