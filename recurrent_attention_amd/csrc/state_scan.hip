// state_scan.hip -- joins the per-segment states of a prefill: a scan of
// S_in[j+1] = a_j * S_in[j] + U_j over the segments of each (b,h), the
// associative composition of the recurrence over consecutive token ranges
// (run from the last segment to the first for the state gradient).
#include "chunk_kernel.h"

namespace la {

template <bool REV>
hipError_t launch_state_scan_dir(const ChunkParams& p, int dk, int dv, hipStream_t s) {
    const int nbx = (dk * dv / 4 + 255) / 256;
    const dim3 grid((unsigned)(nbx * p.BH)), block(256);
    if (dk == dv) {
        switch (dk) {
            case 16: LA_LAUNCH((state_scan_kernel<16, 16, REV>), grid, block, s, p); break;
            case 32: LA_LAUNCH((state_scan_kernel<32, 32, REV>), grid, block, s, p); break;
            case 64: LA_LAUNCH((state_scan_kernel<64, 64, REV>), grid, block, s, p); break;
            case 128: LA_LAUNCH((state_scan_kernel<128, 128, REV>), grid, block, s, p); break;
            default: return hipErrorInvalidValue;
        }
    } else if (dk == 64 && dv == 128) {
        LA_LAUNCH((state_scan_kernel<64, 128, REV>), grid, block, s, p);
    } else if (dk == 128 && dv == 64) {
        LA_LAUNCH((state_scan_kernel<128, 64, REV>), grid, block, s, p);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_state_scan(const ChunkParams& p, int dk, int dv, bool rev, hipStream_t s) {
    return rev ? launch_state_scan_dir<true>(p, dk, dv, s) : launch_state_scan_dir<false>(p, dk, dv, s);
}

}  // namespace la
