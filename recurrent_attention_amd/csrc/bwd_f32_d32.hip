// bwd_f32_d32.hip -- chunkwise backward kernels for d_k = d_v = 32, fp32 inputs.
#include "bwd_kernel.h"

namespace la {
LA_DEFINE_BWD_LAUNCHER(launch_bwd_f32_d32, 32, false)
}  // namespace la
