// chunk_bf16_d128.hip -- chunkwise prefill kernels for d_k = d_v = 128, bf16 inputs.
#include "chunk_kernel.h"

namespace la {
LA_DEFINE_CHUNK_LAUNCHER(launch_chunk_bf16_d128, 128, true)
}  // namespace la
