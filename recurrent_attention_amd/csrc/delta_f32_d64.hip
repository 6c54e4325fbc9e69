// delta_f32_d64.hip -- delta-rule kernels for d_k = d_v = 64, fp32 inputs.
#include "delta_kernel.h"

namespace la {
LA_DEFINE_DELTA_LAUNCHER(launch_delta_f32_d64, 64, false)
}  // namespace la
