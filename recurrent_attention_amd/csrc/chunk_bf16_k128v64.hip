// chunk_bf16_k128v64.hip -- chunkwise prefill kernels for d_k = 128, d_v = 64, bf16 inputs.
#include "chunk_kernel.h"

namespace la {
LA_DEFINE_CHUNK_LAUNCHER_KV(launch_chunk_bf16_k128v64, 128, 64, true)
}  // namespace la
