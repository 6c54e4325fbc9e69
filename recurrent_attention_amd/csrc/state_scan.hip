// state_scan.hip -- joins the per-segment states of a prefill: a scan of
// S_in[j+1] = a_j * S_in[j] + U_j over the segments of each (b,h), the
// associative composition of the recurrence over consecutive token ranges.
#include "chunk_kernel.h"

namespace la {

hipError_t launch_state_scan(const ChunkParams& p, int d, hipStream_t s) {
    const int nbx = (d * d / 4 + 255) / 256;
    const dim3 grid((unsigned)(nbx * p.BH)), block(256);
    switch (d) {
        case 16: hipLaunchKernelGGL((state_scan_kernel<16, 16>), grid, block, 0, s, p); break;
        case 32: hipLaunchKernelGGL((state_scan_kernel<32, 32>), grid, block, 0, s, p); break;
        case 64: hipLaunchKernelGGL((state_scan_kernel<64, 64>), grid, block, 0, s, p); break;
        case 128: hipLaunchKernelGGL((state_scan_kernel<128, 128>), grid, block, 0, s, p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace la
