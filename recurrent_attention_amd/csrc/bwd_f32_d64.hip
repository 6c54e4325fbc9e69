// bwd_f32_d64.hip -- chunkwise backward kernels for d_k = d_v = 64, fp32 inputs.
#include "bwd_kernel.h"

namespace la {
LA_DEFINE_BWD_LAUNCHER(launch_bwd_f32_d64, 64, false)
}  // namespace la
