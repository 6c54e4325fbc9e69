// chunk_bf16_d64.hip -- chunkwise prefill kernels for d_k = d_v = 64, bf16 inputs.
#include "chunk_kernel.h"

namespace la {
LA_DEFINE_CHUNK_LAUNCHER(launch_chunk_bf16_d64, 64, true)
}  // namespace la
