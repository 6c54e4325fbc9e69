// delta_f32_d128.hip -- delta-rule kernels for d_k = d_v = 128, fp32 inputs.
#include "delta_kernel.h"

namespace la {
LA_DEFINE_DELTA_LAUNCHER(launch_delta_f32_d128, 128, false)
}  // namespace la
