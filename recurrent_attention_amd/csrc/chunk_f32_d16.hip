// chunk_f32_d16.hip -- chunkwise prefill kernels for d_k = d_v = 16, f32 inputs.
#include "chunk_kernel.h"

namespace la {
LA_DEFINE_CHUNK_LAUNCHER(launch_chunk_f32_d16, 16, false)
}  // namespace la
