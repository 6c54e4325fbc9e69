// chunk_f32_d32.hip -- chunkwise prefill kernels for d_k = d_v = 32, f32 inputs.
#include "chunk_kernel.h"

namespace la {
LA_DEFINE_CHUNK_LAUNCHER(launch_chunk_f32_d32, 32, false)
}  // namespace la
