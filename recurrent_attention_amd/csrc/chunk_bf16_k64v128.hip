// chunk_bf16_k64v128.hip -- chunkwise prefill kernels for d_k = 64, d_v = 128, bf16 inputs.
#include "chunk_kernel.h"

namespace la {
LA_DEFINE_CHUNK_LAUNCHER_KV(launch_chunk_bf16_k64v128, 64, 128, true)
}  // namespace la
