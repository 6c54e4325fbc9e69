// la_internal.h -- parameter blocks passed by value from the host API to the
// kernels, and the launch entry points each kernel file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/la.h"

namespace la {

// Prefill (chunkwise) parameters; one block serves the state pass, the main
// pass and the segment scan.
struct ChunkParams {
    const void* q;          // [BH, L, dk] dtype
    const void* k;          // [BH, L, dk] dtype
    const void* v;          // [BH, L, dv] dtype
    const float* log_alpha; // [BH, L, dk] (DIAG)
    const float* S0;        // [BH, dk, dv] or null (zeros)
    const float* z0;        // [BH, dk] or null
    void* out;              // [BH, L, dv] dtype
    float* S_final;         // [BH, dk, dv] or null
    float* z_final;         // [BH, dk] or null
    float* ws_S;            // [BH, P, dk*dv] segment states (P > 1)
    float* ws_a;            // [BH, P, dk]    segment decay products
    float* ws_z;            // [BH, P, dk]    segment normaliser parts
    int L, H, BH;
    int P;                  // segments per (b,h)
    int cps;                // chunks per segment (last one may be shorter)
    int nchunks;            // ceil(L / C)
    int phi_elu1, normalize;
    float log2_gamma[LA_MAX_GAMMA_HEADS];  // GAMMA: log2(gamma_h), -inf for 0
};

struct DecodeParams {
    const void* q;          // [BH, dk]
    const void* k;          // [BH, dk]
    const void* v;          // [BH, dv]
    const float* log_alpha; // [BH, dk] (DIAG)
    float* S;               // [BH, dk, dv]
    float* z;               // [BH, dk] or null
    void* out;              // [BH, dv]
    int H, BH;
    int phi_elu1, normalize;
    float gamma[LA_MAX_GAMMA_HEADS];
};

// Kernel families, as named by the profiling interface.
enum KernelId { K_CHUNK_MAIN = 0, K_CHUNK_STATE = 1, K_STATE_SCAN = 2, K_DECODE = 3, K_COUNT = 4 };

// Launch hooks implemented in the kernel files.  Each returns hipSuccess or
// the launch error; shapes have been validated by the caller.  The chunk
// launchers take `sonly` = true for the state pass and `nblocks` workgroups.
#define LA_DECLARE_CHUNK_LAUNCHER(NAME) \
    hipError_t NAME(const ChunkParams& p, int chunk, int gate, bool sonly, hipStream_t s, int nblocks);
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d16)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d32)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d64)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d128)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_d32)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_d64)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_d128)
#undef LA_DECLARE_CHUNK_LAUNCHER
hipError_t launch_state_scan(const ChunkParams& p, int d, hipStream_t s);
hipError_t launch_decode(const DecodeParams& p, int d, bool bf16, int gate, hipStream_t s);

}  // namespace la
