// bwd_bf16_d64.hip -- chunkwise backward kernels for d_k = d_v = 64, bf16 inputs.
#include "bwd_kernel.h"

namespace la {
LA_DEFINE_BWD_LAUNCHER(launch_bwd_bf16_d64, 64, true)
}  // namespace la
