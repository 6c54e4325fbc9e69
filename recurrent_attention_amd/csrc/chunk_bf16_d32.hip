// chunk_bf16_d32.hip -- chunkwise prefill kernels for d_k = d_v = 32, bf16 inputs.
#include "chunk_kernel.h"

namespace la {
LA_DEFINE_CHUNK_LAUNCHER(launch_chunk_bf16_d32, 32, true)
}  // namespace la
