// la_internal.h -- parameter blocks passed by value from the host API to the
// kernels, and the launch entry points each kernel file provides.
#pragma once

#include <hip/hip_ext.h>
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
    int* slow_flags;        // [BH, P] vector-gate main pass: segments handed to the sub-chunk kernel
    const int* cu_seqlens;  // packed sequences: [B + 1] token offsets into each head's L tokens, or null
    const int* seq_order;   // packed sequences: the launch order of the sequences (a permutation of [0, B)), or null
    const float* gn_w;      // output group norm: per-channel scale [H, dv] or null (ones)
    const float* gn_b;      //   per-channel shift [H, dv] or null (zeros)
    const void* gn_gate;    //   swish gate [BH, L, dv] dtype, or null
    float gn_eps;
    void* st_rows;          // backward: state at every chunk boundary [BH, st_slots, dk, dv] dtype
    int st_slots;           // boundary slots per (b,h)
    int L, H, BH;
    int P;                  // segments per (b,h)
    int cps;                // chunks per segment (last one may be shorter)
    int nchunks;            // ceil(L / C)
    int chunk;              // C, the chunk length: at most the kernel's tile, the rest of a
                            // tile masked
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

// Backward (chunkwise) parameters: one workgroup per (b,h, chunk).
struct BwdParams {
    const void* q;          // [BH, L, d] dtype
    const void* k;          // [BH, L, d] dtype
    const void* v;          // [BH, L, d] dtype
    const void* dout;       // [BH, L, d] dtype
    const float* log_alpha; // [BH, L, d] (DIAG)
    const void* st_fwd;     // [BH, nchunks + 1, d, d] dtype: state before each chunk, then the final state
    const float* g_entry;   // [BH, P, d, d]: gradient of the state after each segment's last chunk, or null (zeros)
    float* dS0;             // [BH, d, d]: gradient of the initial state, or null
    void* dq;               // [BH, L, d] dtype
    void* dk;               // [BH, L, d] dtype
    void* dv;               // [BH, L, d] dtype
    float* dlog_alpha;      // [BH, L, d] (DIAG)
    int L, H, BH;
    int nchunks;
    int P, cps;             // segments per (b,h) and chunks per segment
    int phi_elu1;
    float log2_gamma[LA_MAX_GAMMA_HEADS];
};

// Delta rule parameters (prefill and decode).
struct DeltaParams {
    const void* q;          // prefill [BH, L, d], decode [BH, d] dtype
    const void* k;
    const void* v;
    const float* beta;      // prefill [BH, L], decode [BH]
    const float* S0;        // prefill: [BH, d, d] or null (zeros)
    void* out;              // prefill [BH, L, d], decode [BH, d] dtype
    float* S_final;         // prefill: [BH, d, d] or null
    float* S;               // decode: [BH, d, d], updated in place
    int L, H, BH;
};

// Passes of the chunk kernel.  MAIN and STATE serve the forward; the
// backward adds the reversed state pass (segment aggregates of the state
// gradient) and the pass that stores the state at every chunk boundary.
enum ChunkPass {
    PASS_MAIN = 0, PASS_STATE = 1, PASS_STATE_REV = 2, PASS_STORE = 3,
    PASS_MAIN_NORM = 5,  // main pass with the group-norm / swish-gate output epilogue (chunk 64)
    PASS_MAIN_STORE = 6  // main pass that also stores the state at every chunk boundary
};

// Whether the prefill builds the 128-token tile (chunks of 80 to 128
// tokens) for this width and element type: its q, k, K^T, V^T and score
// tiles fit the 160 KiB of LDS for bf16 at d <= 64 and fp32 at d <= 32.
template <int D, bool BF> constexpr bool chunk_tile128() { return BF ? D <= 64 : D <= 32; }
inline bool chunk_tile128_rt(int d, bool bf) { return bf ? d <= 64 : d <= 32; }

// Chunk length of the backward: 64 tokens, 32 for fp32 at d = 128 (whose
// six tiles of 64 tokens would not fit in the 160 KiB of LDS).
constexpr int bwd_chunk(int d, bool bf16) { return (!bf16 && d >= 128) ? 32 : 64; }

// Kernel families, as named by the profiling interface.
enum KernelId {
    K_CHUNK_MAIN = 0, K_CHUNK_STATE = 1, K_STATE_SCAN = 2, K_DECODE = 3,
    K_CHUNK_STORE = 4, K_BWD = 5, K_DELTA = 6, K_DELTA_DECODE = 7, K_SEQ_ORDER = 8,
    K_CHUNK_SUB = 9, K_COUNT = 10
};

// Event pair that the library's launches record around their kernel while
// it profiles (hipExtLaunchKernel takes the timestamps from the kernel's own
// dispatch, so no marker packet sits between an event and its kernel), or
// nulls: set by the host API around one launch, per calling thread.
struct LaunchEvents {
    hipEvent_t start = nullptr, stop = nullptr;
};
LaunchEvents& launch_events();

#define LA_LAUNCH(KERNEL, GRID, BLOCK, S, ...)                                                    \
    do {                                                                                          \
        const ::la::LaunchEvents& la_ev_ = ::la::launch_events();                                 \
        if (la_ev_.start)                                                                         \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, S, la_ev_.start, la_ev_.stop, 0,        \
                                  __VA_ARGS__);                                                   \
        else                                                                                      \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, S, __VA_ARGS__);                           \
    } while (0)

// Launch hooks implemented in the kernel files.  Each returns hipSuccess or
// the launch error; shapes have been validated by the caller.  The chunk
// launchers take the pass (ChunkPass) and `nblocks` workgroups.
#define LA_DECLARE_CHUNK_LAUNCHER(NAME) \
    hipError_t NAME(const ChunkParams& p, int chunk, int gate, int pass, hipStream_t s, int nblocks, \
                    bool robust);
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d16)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d32)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d64)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_f32_d128)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_d32)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_d64)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_d128)
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_k64v128)    // d_k = 64, d_v = 128
LA_DECLARE_CHUNK_LAUNCHER(launch_chunk_bf16_k128v64)    // d_k = 128, d_v = 64
#undef LA_DECLARE_CHUNK_LAUNCHER
hipError_t launch_state_scan(const ChunkParams& p, int dk, int dv, bool rev, hipStream_t s);
// Packed sequences: order[0..B) = the sequences by decreasing chunk count.
hipError_t launch_seq_order(const int* cu_seqlens, int B, int T, int chunk, int max_seqlen,
                            int* order, hipStream_t s);
#define LA_DECLARE_DELTA_LAUNCHER(NAME) \
    hipError_t NAME(const DeltaParams& p, bool decode, hipStream_t s);
LA_DECLARE_DELTA_LAUNCHER(launch_delta_f32_d16)
LA_DECLARE_DELTA_LAUNCHER(launch_delta_f32_d32)
LA_DECLARE_DELTA_LAUNCHER(launch_delta_f32_d64)
LA_DECLARE_DELTA_LAUNCHER(launch_delta_f32_d128)
LA_DECLARE_DELTA_LAUNCHER(launch_delta_bf16_d32)
LA_DECLARE_DELTA_LAUNCHER(launch_delta_bf16_d64)
LA_DECLARE_DELTA_LAUNCHER(launch_delta_bf16_d128)
#undef LA_DECLARE_DELTA_LAUNCHER
#define LA_DECLARE_BWD_LAUNCHER(NAME) \
    hipError_t NAME(const BwdParams& p, int gate, hipStream_t s);
LA_DECLARE_BWD_LAUNCHER(launch_bwd_f32_d16)
LA_DECLARE_BWD_LAUNCHER(launch_bwd_f32_d32)
LA_DECLARE_BWD_LAUNCHER(launch_bwd_f32_d64)
LA_DECLARE_BWD_LAUNCHER(launch_bwd_f32_d128)
LA_DECLARE_BWD_LAUNCHER(launch_bwd_bf16_d32)
LA_DECLARE_BWD_LAUNCHER(launch_bwd_bf16_d64)
LA_DECLARE_BWD_LAUNCHER(launch_bwd_bf16_d128)
#undef LA_DECLARE_BWD_LAUNCHER
hipError_t launch_decode(const DecodeParams& p, int dk, int dv, bool bf16, int gate, hipStream_t s);

}  // namespace la
