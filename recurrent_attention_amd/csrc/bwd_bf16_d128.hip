// bwd_bf16_d128.hip -- chunkwise backward kernels for d_k = d_v = 128, bf16 inputs.
#include "bwd_kernel.h"

namespace la {
LA_DEFINE_BWD_LAUNCHER(launch_bwd_bf16_d128, 128, true)
}  // namespace la
