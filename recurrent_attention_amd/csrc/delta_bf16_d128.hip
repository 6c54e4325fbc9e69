// delta_bf16_d128.hip -- delta-rule kernels for d_k = d_v = 128, bf16 inputs.
#include "delta_kernel.h"

namespace la {
LA_DEFINE_DELTA_LAUNCHER(launch_delta_bf16_d128, 128, true)
}  // namespace la
