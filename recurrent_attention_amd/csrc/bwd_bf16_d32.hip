// bwd_bf16_d32.hip -- chunkwise backward kernels for d_k = d_v = 32, bf16 inputs.
#include "bwd_kernel.h"

namespace la {
LA_DEFINE_BWD_LAUNCHER(launch_bwd_bf16_d32, 32, true)
}  // namespace la
