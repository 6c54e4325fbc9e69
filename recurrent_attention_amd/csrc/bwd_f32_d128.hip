// bwd_f32_d128.hip -- chunkwise backward kernels for d_k = d_v = 128, fp32 inputs.
#include "bwd_kernel.h"

namespace la {
LA_DEFINE_BWD_LAUNCHER(launch_bwd_f32_d128, 128, false)
}  // namespace la
