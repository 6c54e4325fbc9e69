// la_api.hip -- host side of the C ABI declared in include/la.h: argument
// validation, the choice of sequence segments, launch sequencing and the
// optional per-kernel event timing.  Nothing here allocates device memory or
// synchronises outside the profiling query.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "la_internal.h"

namespace la {
LaunchEvents& launch_events() {
    static thread_local LaunchEvents ev;
    return ev;
}
}  // namespace la

namespace {

thread_local char g_errmsg[512] = "";

la_status fail(la_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_errmsg, sizeof g_errmsg, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups the automatic segment choice aims for: one per compute unit of
// an MI355X (256 CUs).
constexpr int kTargetBlocks = 256;
// Fewest chunks the automatic choice gives a segment: below that the state
// pass and the scan (two more launches) cost more than the shorter walk
// saves (a 4-chunk sequence runs in one launch).
constexpr int kMinSegmentChunks = 4;

struct Plan {
    int nchunks, P, cps;
};

Plan make_plan(const la_desc* d, int chunk) {
    Plan pl;
    pl.nchunks = (d->L + chunk - 1) / chunk;
    const long bh = (long)d->B * d->H;
    int P = d->segments;
    if (P <= 0) {
        P = (int)((kTargetBlocks + bh - 1) / bh);
        if (P > pl.nchunks / kMinSegmentChunks) P = pl.nchunks / kMinSegmentChunks;
    }
    if (P < 1) P = 1;
    if (P > pl.nchunks) P = pl.nchunks;
    pl.cps = (pl.nchunks + P - 1) / P;
    pl.P = (pl.nchunks + pl.cps - 1) / pl.cps;  // every segment non-empty
    return pl;
}

size_t align16(size_t n) { return (n + 15) & ~(size_t)15; }

// Segment slots (states, decays, normaliser parts; several segments only),
// rounded up to 16 bytes.
size_t slot_bytes(const la_desc* d, const Plan& pl) {
    if (pl.P <= 1) return 0;
    const size_t slots = (size_t)d->B * d->H * pl.P;
    return align16(slots * ((size_t)d->dk * d->dv + 2 * (size_t)d->dk) * sizeof(float));
}
// One int32 per (b,h) segment: under a vector gate, whether the main pass
// handed the segment to the sub-chunk kernel.
size_t flag_bytes(const la_desc* d, const Plan& pl) {
    return align16((size_t)d->B * d->H * pl.P * sizeof(int));
}
size_t workspace_bytes(const la_desc* d, const Plan& pl) { return slot_bytes(d, pl) + flag_bytes(d, pl); }

// Packed sequences: after the segment slots and flags, the launch order of
// the sequences (int32 [B], rounded up to 16 bytes).
size_t order_bytes(const la_desc* d) { return align16((size_t)d->B * sizeof(int)); }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
// d_k != d_v: 64 and 128 either way (prefill in bf16, decode in both types)
bool mixed_pair(const la_desc* d) {
    return (d->dk == 64 && d->dv == 128) || (d->dk == 128 && d->dv == 64);
}
// Chunk lengths of the prefill: multiples of 16 from 16 to 128; above 64
// only where the 128-token tile is built (d_k == d_v).
bool supported_chunk(const la_desc* d, int c) {
    if (c < 16 || c > 128 || c % 16 != 0) return false;
    return c <= 64 || (d->dk == d->dv && la::chunk_tile128_rt(d->dk, d->dtype == LA_BF16));
}
la_status check_chunk(const la_desc* d, int c) {
    if (c < 16 || c > 128 || c % 16 != 0)
        return fail(LA_ERR_UNSUPPORTED, "chunk must be a multiple of 16 in [16, 128] (got %d)", c);
    if (!supported_chunk(d, c))
        return fail(LA_ERR_UNSUPPORTED,
                    "chunks above 64 are built for dk == dv, bf16 at dk <= 64 and fp32 at "
                    "dk <= 32 (chunk %d, dk %d, dv %d)", c, d->dk, d->dv);
    return LA_OK;
}

// mfma: the shape runs on matrix cores (every prefill-like path), where
// bf16 operands need d_k >= 32; the decode step streams the state on the
// vector units and takes bf16 at every built width.  mixed: the entry point
// is built for d_k != d_v (the prefill in bf16, the decode step).
la_status check_desc(const la_desc* d, bool mfma = true, bool mixed = false) {
    if (!d) return fail(LA_ERR_INVALID, "descriptor is NULL");
    if (d->B < 1 || d->H < 1 || d->L < 1 || d->dk < 1 || d->dv < 1)
        return fail(LA_ERR_INVALID, "dimensions must be >= 1 (B=%d H=%d L=%d dk=%d dv=%d)", d->B,
                    d->H, d->L, d->dk, d->dv);
    if (d->dtype != LA_F32 && d->dtype != LA_BF16)
        return fail(LA_ERR_INVALID, "unknown dtype %d", d->dtype);
    if (d->phi != LA_PHI_IDENTITY && d->phi != LA_PHI_ELU1)
        return fail(LA_ERR_INVALID, "unknown feature map %d", d->phi);
    if (d->normalize != 0 && d->normalize != 1)
        return fail(LA_ERR_INVALID, "normalize must be 0 or 1");
    if (d->segments < 0) return fail(LA_ERR_INVALID, "segments must be >= 0");
    if ((long long)d->B * d->H > (1LL << 24))
        return fail(LA_ERR_UNSUPPORTED, "B*H = %lld exceeds 2^24", (long long)d->B * d->H);
    if (!supported_d(d->dk) || !supported_d(d->dv) ||
        (d->dk != d->dv && !(mixed && mixed_pair(d) && (d->dtype == LA_BF16 || !mfma))))
        return fail(LA_ERR_UNSUPPORTED,
                    "built shapes: dk == dv in {16,32,64,128}; dk, dv = 64, 128 either way for the "
                    "bf16 prefill and the decode step (dk=%d dv=%d)", d->dk, d->dv);
    if (mfma && d->dtype == LA_BF16 && d->dk < 32)
        return fail(LA_ERR_UNSUPPORTED, "bf16 prefill inputs need dk >= 32 (dk=%d)", d->dk);
    // kernels address one (b,h) slice of a tensor with 32-bit byte offsets
    if ((long long)d->L * (d->dk > d->dv ? d->dk : d->dv) * 4 > 0xFFFFFFFFLL)
        return fail(LA_ERR_UNSUPPORTED, "L*d*4 must stay below 2^32 bytes (L=%d)", d->L);
    return LA_OK;
}

// Gates read from device memory (one per token and channel, or per token).
bool device_gate(int gate_mode) { return gate_mode == LA_GATE_DIAG || gate_mode == LA_GATE_SCALAR; }

la_status check_gate(const la_desc* d, int gate_mode, const float* g, bool device_diag,
                     float* log2_gamma, float* gamma) {
    if (gate_mode == LA_GATE_NONE) return LA_OK;
    if (gate_mode == LA_GATE_GAMMA) {
        if (!g) return fail(LA_ERR_INVALID, "GAMMA gate needs a host gamma[H] array");
        if (d->H > LA_MAX_GAMMA_HEADS)
            return fail(LA_ERR_UNSUPPORTED, "GAMMA gate supports at most %d heads (H=%d)",
                        LA_MAX_GAMMA_HEADS, d->H);
        for (int h = 0; h < d->H; ++h) {
            const float x = g[h];
            if (!(x >= 0.0f && x <= 1.0f))
                return fail(LA_ERR_INVALID, "gamma[%d] = %g is outside [0, 1]", h, (double)x);
            if (log2_gamma) log2_gamma[h] = x > 0.0f ? (float)std::log2((double)x) : -INFINITY;
            if (gamma) gamma[h] = x;
        }
        return LA_OK;
    }
    if (gate_mode == LA_GATE_DIAG || gate_mode == LA_GATE_SCALAR) {
        if (!g) return fail(LA_ERR_INVALID, "%s gate needs a device log-gate array",
                            gate_mode == LA_GATE_DIAG ? "DIAG" : "SCALAR");
        if (device_diag && !aligned16(g)) return fail(LA_ERR_INVALID, "log-gate pointer is not 16-byte aligned");
        return LA_OK;
    }
    return fail(LA_ERR_INVALID, "unknown gate mode %d", gate_mode);
}

// ------------------------------------------------------------------ profiling
struct ProfRec {
    int kernel;
    hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

const char* kKernelNames[la::K_COUNT] = {"chunk_main", "chunk_state", "state_scan", "decode",
                                         "chunk_store", "chunk_bwd", "delta_chunk",
                                         "delta_decode", "seq_order", "chunk_sub"};

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Wraps one launch; while profiling, the launch records an event pair
// around its kernel (la::LA_LAUNCH).
template <class F>
hipError_t timed_launch(int kernel, hipStream_t s, F&& launch) {
    (void)s;
    std::unique_lock<std::mutex> lk(g_prof_mu);
    if (!g_prof_on) {
        lk.unlock();
        return launch();
    }
    ProfRec rec{kernel, take_event(), take_event()};
    if (!rec.a || !rec.b) return hipErrorOutOfMemory;
    la::launch_events() = la::LaunchEvents{rec.a, rec.b};
    const hipError_t e = launch();
    la::launch_events() = la::LaunchEvents{};
    if (e != hipSuccess) return e;
    g_prof.push_back(rec);
    return hipSuccess;
}

hipError_t chunk_launch(const la_desc* d, const la::ChunkParams& p, int chunk, int gate, int pass,
                        hipStream_t s, int nblocks, bool robust = false) {
    const bool bf16 = d->dtype == LA_BF16;
    if (d->dk != d->dv)
        return d->dk == 64 ? la::launch_chunk_bf16_k64v128(p, chunk, gate, pass, s, nblocks, robust)
                           : la::launch_chunk_bf16_k128v64(p, chunk, gate, pass, s, nblocks, robust);
    switch (d->dk) {
        case 16: return la::launch_chunk_f32_d16(p, chunk, gate, pass, s, nblocks, robust);
        case 32: return bf16 ? la::launch_chunk_bf16_d32(p, chunk, gate, pass, s, nblocks, robust)
                             : la::launch_chunk_f32_d32(p, chunk, gate, pass, s, nblocks, robust);
        case 64: return bf16 ? la::launch_chunk_bf16_d64(p, chunk, gate, pass, s, nblocks, robust)
                             : la::launch_chunk_f32_d64(p, chunk, gate, pass, s, nblocks, robust);
        default: return bf16 ? la::launch_chunk_bf16_d128(p, chunk, gate, pass, s, nblocks, robust)
                             : la::launch_chunk_f32_d128(p, chunk, gate, pass, s, nblocks, robust);
    }
}

hipError_t delta_launch(const la_desc* d, const la::DeltaParams& p, bool decode, hipStream_t s) {
    const bool bf16 = d->dtype == LA_BF16;
    switch (d->dk) {
        case 16: return la::launch_delta_f32_d16(p, decode, s);
        case 32: return bf16 ? la::launch_delta_bf16_d32(p, decode, s) : la::launch_delta_f32_d32(p, decode, s);
        case 64: return bf16 ? la::launch_delta_bf16_d64(p, decode, s) : la::launch_delta_f32_d64(p, decode, s);
        default: return bf16 ? la::launch_delta_bf16_d128(p, decode, s) : la::launch_delta_f32_d128(p, decode, s);
    }
}

// Shape checks shared by the delta-rule entry points: no feature map, no
// normaliser (the rule has neither).
la_status check_delta(const la_desc* d) {
    const la_status st = check_desc(d);
    if (st != LA_OK) return st;
    if (d->phi != LA_PHI_IDENTITY)
        return fail(LA_ERR_UNSUPPORTED, "the delta rule takes its keys as given (phi must be identity)");
    if (d->normalize) return fail(LA_ERR_UNSUPPORTED, "the delta rule has no normaliser");
    return LA_OK;
}

hipError_t bwd_launch(const la_desc* d, const la::BwdParams& p, int gate, hipStream_t s) {
    const bool bf16 = d->dtype == LA_BF16;
    switch (d->dk) {
        case 16: return la::launch_bwd_f32_d16(p, gate, s);
        case 32: return bf16 ? la::launch_bwd_bf16_d32(p, gate, s) : la::launch_bwd_f32_d32(p, gate, s);
        case 64: return bf16 ? la::launch_bwd_bf16_d64(p, gate, s) : la::launch_bwd_f32_d64(p, gate, s);
        default: return bf16 ? la::launch_bwd_bf16_d128(p, gate, s) : la::launch_bwd_f32_d128(p, gate, s);
    }
}

// Backward workspace, in bytes: the state before every chunk and the final
// state in the element type of q/k/v, then the fp32 segment slots of the
// state passes.
struct BwdLayout {
    size_t fwd, seg, total;
};
BwdLayout bwd_layout(const la_desc* d, const Plan& pl) {
    const size_t bh = (size_t)d->B * d->H, dd = (size_t)d->dk * d->dv;
    const size_t es = d->dtype == LA_BF16 ? 2 : 4;
    BwdLayout w;
    w.fwd = 0;
    w.seg = w.fwd + bh * (pl.nchunks + 1) * dd * es;
    w.total = w.seg + (pl.P > 1 ? bh * pl.P * (dd + 2 * (size_t)d->dk) * sizeof(float) : 0);
    return w;
}

// The descriptor the segment plan is made for: packed sequences plan for the
// longest one (every sequence gets the same number of segments; those past
// a shorter sequence's end are empty and compose as the identity).
la_desc plan_desc(const la_desc* d, bool packed, int max_seqlen) {
    la_desc dp = *d;
    if (packed) dp.L = max_seqlen;
    return dp;
}

la_status check_varlen(const la_desc* d, const int* cu_seqlens, int max_seqlen) {
    const la_status st = check_desc(d, true, true);
    if (st != LA_OK) return st;
    if (!cu_seqlens) return fail(LA_ERR_INVALID, "cu_seqlens must be non-NULL");
    if (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)
        return fail(LA_ERR_INVALID, "cu_seqlens must be 4-byte aligned");
    if (max_seqlen < 1 || max_seqlen > d->L)
        return fail(LA_ERR_INVALID, "max_seqlen=%d must be in [1, L=%d]", max_seqlen, d->L);
    return LA_OK;
}

la_status hip_fail(hipError_t e, const char* what) {
    return fail(LA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ------------------------------------------------------------ no-alloc scratch
// The segment workspace of la_chunk_fwd_noalloc: one copy per GPU, held for
// the life of the process.  In host code `scratch` only names the symbol; its
// device address (a different one on every GPU) comes from
// hipGetSymbolAddress with that GPU current, and only that address is ever
// handed to a kernel.
static __device__ __align__(256) unsigned char scratch[LA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of `scratch` on the GPU that `s` belongs to (the current
// GPU for the null stream), looked up once per GPU.
la_status scratch_address(hipStream_t s, void** out) {
    int dev = -1;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return fail(LA_ERR_HIP, "device of the stream: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(LA_ERR_UNSUPPORTED, "device %d is beyond the %d the scratch table holds", dev,
                    kMaxScratchDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return fail(LA_ERR_HIP, "current device: %s", hipGetErrorString(e));
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return fail(LA_ERR_HIP, "select device %d: %s", dev, hipGetErrorString(e));
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
        if (e != hipSuccess || !ptr)
            return fail(LA_ERR_HIP, "scratch address on device %d: %s", dev,
                        hipGetErrorString(e != hipSuccess ? e : hipErrorInvalidSymbol));
        if (e2 != hipSuccess)
            return fail(LA_ERR_HIP, "restore device %d: %s", cur, hipGetErrorString(e2));
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LA_OK;
}

// use_scratch: take the workspace from the static scratch array (after all
// validation, so an invalid call makes no HIP call at all)
la_status chunk_fwd_impl(const la_desc* d, const int* cu_seqlens, int max_seqlen, const void* q,
                         const void* k, const void* v, int gate_mode,
                         const float* gamma_or_log_alpha, const float* S0, const float* z0,
                         int chunk, const la_groupnorm* gn, void* out, float* S_final,
                         float* z_final, void* workspace, size_t ws_bytes, void* stream,
                         void* states = nullptr, bool use_scratch = false) {
    // packed sequences plan their segments for the longest one
    const la_desc dp = plan_desc(d, cu_seqlens != nullptr, max_seqlen);
    la_status st;
    st = check_chunk(d, chunk);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !out) return fail(LA_ERR_INVALID, "q, k, v and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
        (S0 && !aligned16(S0)) || (z0 && !aligned16(z0)) || (S_final && !aligned16(S_final)) ||
        (z_final && !aligned16(z_final)))
        return fail(LA_ERR_INVALID, "device pointers must be 16-byte aligned");
    if (!d->normalize && (z0 || z_final))
        return fail(LA_ERR_INVALID, "z0/z_final given without normalize");
    if (d->segments > 0 && d->segments > (dp.L + chunk - 1) / chunk)
        return fail(LA_ERR_INVALID, "segments=%d exceeds the %d chunks", d->segments,
                    (dp.L + chunk - 1) / chunk);
    if (gn) {
        if (chunk != 64) return fail(LA_ERR_UNSUPPORTED, "the group-norm epilogue is built for chunk 64");
        if (!(gn->eps > 0.0f)) return fail(LA_ERR_INVALID, "group-norm eps must be > 0");
        if ((gn->weight && !aligned16(gn->weight)) || (gn->bias && !aligned16(gn->bias)) ||
            (gn->gate && !aligned16(gn->gate)))
            return fail(LA_ERR_INVALID, "device pointers must be 16-byte aligned");
    }

    la::ChunkParams p;
    std::memset(&p, 0, sizeof p);
    if (gn) {
        p.gn_w = gn->weight;
        p.gn_b = gn->bias;
        p.gn_gate = gn->gate;
        p.gn_eps = gn->eps;
    }
    st = check_gate(d, gate_mode, gamma_or_log_alpha, true, p.log2_gamma, nullptr);
    if (st != LA_OK) return st;

    const Plan pl = make_plan(&dp, chunk);
    const size_t seg_bytes = slot_bytes(&dp, pl);
    const size_t flags_at = seg_bytes;
    const size_t order_at = seg_bytes + flag_bytes(&dp, pl);
    const size_t need = order_at + (cu_seqlens ? order_bytes(d) : 0);
    if (use_scratch && need > 0) {
        if (need > LA_NOALLOC_SCRATCH_BYTES)
            return fail(LA_ERR_UNSUPPORTED,
                        "this shape needs %zu bytes of workspace, above the %u of the no-alloc scratch",
                        need, (unsigned)LA_NOALLOC_SCRATCH_BYTES);
        st = scratch_address(static_cast<hipStream_t>(stream), &workspace);
        if (st != LA_OK) return st;
        ws_bytes = LA_NOALLOC_SCRATCH_BYTES;
    }
    if (need > 0) {
        if (!workspace) return fail(LA_ERR_INVALID, "workspace of %zu bytes is required", need);
        if (!aligned16(workspace)) return fail(LA_ERR_INVALID, "workspace must be 16-byte aligned");
        if (ws_bytes < need)
            return fail(LA_ERR_INVALID, "workspace has %zu bytes, %zu required", ws_bytes, need);
    }

    const int BH = d->B * d->H;
    p.q = q;
    p.k = k;
    p.v = v;
    p.log_alpha = device_gate(gate_mode) ? gamma_or_log_alpha : nullptr;
    p.S0 = S0;
    p.z0 = z0;
    p.out = out;
    p.S_final = S_final;
    p.z_final = z_final;
    p.L = d->L;
    p.H = d->H;
    p.BH = BH;
    p.P = pl.P;
    p.cps = pl.cps;
    p.nchunks = pl.nchunks;
    p.chunk = chunk;
    p.phi_elu1 = d->phi == LA_PHI_ELU1;
    p.normalize = d->normalize;
    p.cu_seqlens = cu_seqlens;
    if (states) {
        p.st_rows = states;
        p.st_slots = pl.nchunks + 1;
    }
    if (pl.P > 1) {
        float* ws = static_cast<float*>(workspace);
        const size_t slots = (size_t)BH * pl.P;
        p.ws_S = ws;
        p.ws_a = ws + slots * d->dk * d->dv;
        p.ws_z = p.ws_a + slots * d->dk;
    }
    p.slow_flags = reinterpret_cast<int*>(static_cast<char*>(workspace) + flags_at);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (cu_seqlens) {
        int* order = reinterpret_cast<int*>(static_cast<char*>(workspace) + order_at);
        e = timed_launch(la::K_SEQ_ORDER, s, [&] {
            return la::launch_seq_order(cu_seqlens, d->B, d->L, chunk, max_seqlen, order, s);
        });
        if (e != hipSuccess) return hip_fail(e, "sequence order launch");
        p.seq_order = order;
    }
    if (pl.P > 1) {
        // state pass over every segment but the last, then the segment scan
        e = timed_launch(la::K_CHUNK_STATE, s, [&] {
            return chunk_launch(d, p, chunk, gate_mode, la::PASS_STATE, s, BH * (pl.P - 1));
        });
        if (e != hipSuccess) return hip_fail(e, "state pass launch");
        e = timed_launch(la::K_STATE_SCAN, s, [&] { return la::launch_state_scan(p, d->dk, d->dv, false, s); });
        if (e != hipSuccess) return hip_fail(e, "segment scan launch");
    }
    const int pass = states ? la::PASS_MAIN_STORE : gn ? la::PASS_MAIN_NORM : la::PASS_MAIN;
    e = timed_launch(la::K_CHUNK_MAIN, s, [&] {
        return chunk_launch(d, p, chunk, gate_mode, pass, s, BH * pl.P);
    });
    if (e != hipSuccess) return hip_fail(e, "main pass launch");
    if (device_gate(gate_mode)) {
        // segments with a chunk whose gates are too strong for the
        // chunk-middle reference, again with the sub-chunk path (every other
        // workgroup reads its flag and exits)
        e = timed_launch(la::K_CHUNK_SUB, s, [&] {
            return chunk_launch(d, p, chunk, gate_mode, pass, s, BH * pl.P, true);
        });
        if (e != hipSuccess) return hip_fail(e, "sub-chunk pass launch");
    }
    return LA_OK;
}

}  // namespace

extern "C" {

const char* la_status_string(la_status s) {
    switch (s) {
        case LA_OK: return "ok";
        case LA_ERR_INVALID: return "invalid argument";
        case LA_ERR_UNSUPPORTED: return "unsupported shape or mode";
        case LA_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* la_last_error_message(void) { return g_errmsg; }

int la_version(void) { return LA_VERSION; }

int la_chunk_fwd_segments(const la_desc* d, int chunk) {
    if (check_desc(d, true, true) != LA_OK || !supported_chunk(d, chunk)) return 0;
    return make_plan(d, chunk).P;
}

size_t la_chunk_fwd_workspace_bytes(const la_desc* d, int chunk) {
    if (check_desc(d, true, true) != LA_OK || !supported_chunk(d, chunk)) return 0;
    return workspace_bytes(d, make_plan(d, chunk));
}

la_status la_chunk_fwd(const la_desc* d, const void* q, const void* k, const void* v,
                       int gate_mode, const float* gamma_or_log_alpha, const float* S0,
                       const float* z0, int chunk, void* out, float* S_final, float* z_final,
                       void* workspace, size_t ws_bytes, void* stream) {
    g_errmsg[0] = '\0';
    const la_status st = check_desc(d, true, true);
    if (st != LA_OK) return st;
    return chunk_fwd_impl(d, nullptr, 0, q, k, v, gate_mode, gamma_or_log_alpha, S0, z0, chunk,
                          nullptr, out, S_final, z_final, workspace, ws_bytes, stream);
}

la_status la_chunk_fwd_noalloc(const la_desc* d, const void* q, const void* k, const void* v,
                               int gate_mode, const float* gamma_or_log_alpha, const float* S0,
                               const float* z0, int chunk, void* out, float* S_final,
                               float* z_final, void* stream) {
    g_errmsg[0] = '\0';
    const la_status st = check_desc(d, true, true);
    if (st != LA_OK) return st;
    return chunk_fwd_impl(d, nullptr, 0, q, k, v, gate_mode, gamma_or_log_alpha, S0, z0, chunk,
                          nullptr, out, S_final, z_final, nullptr, 0, stream, nullptr, true);
}

la_status la_chunk_fwd_groupnorm(const la_desc* d, const void* q, const void* k, const void* v,
                                 int gate_mode, const float* gamma_or_log_alpha, const float* S0,
                                 const float* z0, int chunk, const la_groupnorm* gn, void* out,
                                 float* S_final, float* z_final, void* workspace, size_t ws_bytes,
                                 void* stream) {
    g_errmsg[0] = '\0';
    const la_status st = check_desc(d, true, true);
    if (st != LA_OK) return st;
    if (!gn) return fail(LA_ERR_INVALID, "the group-norm description is NULL");
    return chunk_fwd_impl(d, nullptr, 0, q, k, v, gate_mode, gamma_or_log_alpha, S0, z0, chunk,
                          gn, out, S_final, z_final, workspace, ws_bytes, stream);
}

size_t la_chunk_train_states_bytes(const la_desc* d) {
    if (check_desc(d) != LA_OK) return 0;
    const int chunk = la::bwd_chunk(d->dk, d->dtype == LA_BF16);
    const size_t n = (size_t)(d->L + chunk - 1) / chunk + 1;
    return (size_t)d->B * d->H * n * d->dk * d->dv * (d->dtype == LA_BF16 ? 2 : 4);
}

la_status la_chunk_fwd_train(const la_desc* d, const void* q, const void* k, const void* v,
                             int gate_mode, const float* gamma_or_log_alpha, const float* S0,
                             void* out, float* S_final, void* states, size_t states_bytes,
                             void* workspace, size_t ws_bytes, void* stream) {
    g_errmsg[0] = '\0';
    const la_status st = check_desc(d);
    if (st != LA_OK) return st;
    if (d->normalize) return fail(LA_ERR_UNSUPPORTED, "the training forward has no normaliser");
    if (!states) return fail(LA_ERR_INVALID, "states must be non-NULL");
    if (!aligned16(states)) return fail(LA_ERR_INVALID, "device pointers must be 16-byte aligned");
    if (states_bytes < la_chunk_train_states_bytes(d))
        return fail(LA_ERR_INVALID, "states has %zu bytes, %zu required", states_bytes,
                    la_chunk_train_states_bytes(d));
    const int chunk = la::bwd_chunk(d->dk, d->dtype == LA_BF16);
    return chunk_fwd_impl(d, nullptr, 0, q, k, v, gate_mode, gamma_or_log_alpha, S0, nullptr,
                          chunk, nullptr, out, S_final, nullptr, workspace, ws_bytes, stream,
                          states);
}

la_status la_chunk_fwd_varlen(const la_desc* d, const int* cu_seqlens, int max_seqlen,
                              const void* q, const void* k, const void* v, int gate_mode,
                              const float* gamma_or_log_alpha, const float* S0, const float* z0,
                              int chunk, void* out, float* S_final, float* z_final,
                              void* workspace, size_t ws_bytes, void* stream) {
    g_errmsg[0] = '\0';
    const la_status st = check_varlen(d, cu_seqlens, max_seqlen);
    if (st != LA_OK) return st;
    return chunk_fwd_impl(d, cu_seqlens, max_seqlen, q, k, v, gate_mode, gamma_or_log_alpha, S0,
                          z0, chunk, nullptr, out, S_final, z_final, workspace, ws_bytes, stream);
}

size_t la_chunk_fwd_varlen_workspace_bytes(const la_desc* d, int max_seqlen, int chunk) {
    if (check_desc(d, true, true) != LA_OK || !supported_chunk(d, chunk) || max_seqlen < 1 || max_seqlen > d->L)
        return 0;
    const la_desc dp = plan_desc(d, true, max_seqlen);
    return workspace_bytes(&dp, make_plan(&dp, chunk)) + order_bytes(d);
}

size_t la_chunk_bwd_workspace_bytes(const la_desc* d) {
    if (check_desc(d) != LA_OK) return 0;
    const int chunk = la::bwd_chunk(d->dk, d->dtype == LA_BF16);
    return bwd_layout(d, make_plan(d, chunk)).total;
}

int la_chunk_bwd_chunk(const la_desc* d) {
    if (check_desc(d) != LA_OK) return 0;
    return la::bwd_chunk(d->dk, d->dtype == LA_BF16);
}

la_status la_chunk_bwd(const la_desc* d, const void* q, const void* k, const void* v,
                       const void* dout, int gate_mode, const float* gamma_or_log_alpha,
                       const float* S0, const float* dS_final, const void* states, void* dq,
                       void* dk, void* dv, float* dlog_alpha, float* dS0, void* workspace,
                       size_t ws_bytes, void* stream) {
    g_errmsg[0] = '\0';
    la_status st = check_desc(d);
    if (st != LA_OK) return st;
    if (d->normalize) return fail(LA_ERR_UNSUPPORTED, "the backward has no normaliser (normalize=1)");
    if (!q || !k || !v || !dout || !dq || !dk || !dv)
        return fail(LA_ERR_INVALID, "q, k, v, dout, dq, dk and dv must be non-NULL");
    if (device_gate(gate_mode) && !dlog_alpha)
        return fail(LA_ERR_INVALID, "DIAG and SCALAR gates need dlog_alpha");
    if (!device_gate(gate_mode) && dlog_alpha)
        return fail(LA_ERR_INVALID, "dlog_alpha given without a DIAG or SCALAR gate");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || (dlog_alpha && !aligned16(dlog_alpha)) ||
        (S0 && !aligned16(S0)) || (dS_final && !aligned16(dS_final)) || (dS0 && !aligned16(dS0)) ||
        (states && !aligned16(states)))
        return fail(LA_ERR_INVALID, "device pointers must be 16-byte aligned");
    const int chunk = la::bwd_chunk(d->dk, d->dtype == LA_BF16);
    if (d->segments > 0 && d->segments > (d->L + chunk - 1) / chunk)
        return fail(LA_ERR_INVALID, "segments=%d exceeds the %d chunks", d->segments,
                    (d->L + chunk - 1) / chunk);

    la::ChunkParams p;
    std::memset(&p, 0, sizeof p);
    st = check_gate(d, gate_mode, gamma_or_log_alpha, true, p.log2_gamma, nullptr);
    if (st != LA_OK) return st;
    const Plan pl = make_plan(d, chunk);
    const BwdLayout w = bwd_layout(d, pl);
    if (!workspace) return fail(LA_ERR_INVALID, "workspace of %zu bytes is required", w.total);
    if (!aligned16(workspace)) return fail(LA_ERR_INVALID, "workspace must be 16-byte aligned");
    if (ws_bytes < w.total)
        return fail(LA_ERR_INVALID, "workspace has %zu bytes, %zu required", ws_bytes, w.total);

    const int BH = d->B * d->H;
    char* ws = static_cast<char*>(workspace);
    p.log_alpha = device_gate(gate_mode) ? gamma_or_log_alpha : nullptr;
    p.L = d->L;
    p.H = d->H;
    p.BH = BH;
    p.P = pl.P;
    p.cps = pl.cps;
    p.nchunks = pl.nchunks;
    p.chunk = chunk;
    p.phi_elu1 = d->phi == LA_PHI_ELU1;
    if (pl.P > 1) {
        const size_t slots = (size_t)BH * pl.P;
        p.ws_S = reinterpret_cast<float*>(ws + w.seg);
        p.ws_a = p.ws_S + slots * d->dk * d->dv;
        p.ws_z = p.ws_a + slots * d->dk;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;

    // the states before every chunk: the forward state recurrence, unless
    // the training forward left them behind
    p.q = q;
    p.k = k;
    p.v = v;
    p.S0 = S0;
    p.S_final = nullptr;
    p.st_rows = ws + w.fwd;
    p.st_slots = pl.nchunks + 1;
    if (!states && pl.P > 1) {
        e = timed_launch(la::K_CHUNK_STATE, s, [&] {
            return chunk_launch(d, p, chunk, gate_mode, la::PASS_STATE, s, BH * (pl.P - 1));
        });
        if (e != hipSuccess) return hip_fail(e, "state pass launch");
        e = timed_launch(la::K_STATE_SCAN, s, [&] { return la::launch_state_scan(p, d->dk, d->dv, false, s); });
        if (e != hipSuccess) return hip_fail(e, "segment scan launch");
    }
    if (!states) {
        e = timed_launch(la::K_CHUNK_STORE, s, [&] {
            return chunk_launch(d, p, chunk, gate_mode, la::PASS_STORE, s, BH * pl.P);
        });
        if (e != hipSuccess) return hip_fail(e, "state store launch");
    }

    // the state gradient entering each segment (P > 1): the same recurrence
    // run from the end with phi(q) and dout in the places of phi(k) and v,
    // aggregated per segment and composed from the last segment to the first
    p.k = q;
    p.v = dout;
    p.S0 = dS_final;
    p.S_final = nullptr;
    p.st_rows = nullptr;
    if (pl.P > 1) {
        e = timed_launch(la::K_CHUNK_STATE, s, [&] {
            return chunk_launch(d, p, chunk, gate_mode, la::PASS_STATE_REV, s, BH * (pl.P - 1));
        });
        if (e != hipSuccess) return hip_fail(e, "reverse state pass launch");
        e = timed_launch(la::K_STATE_SCAN, s, [&] { return la::launch_state_scan(p, d->dk, d->dv, true, s); });
        if (e != hipSuccess) return hip_fail(e, "reverse segment scan launch");
    }

    // the gradients: each segment walked from its last chunk to its first,
    // the state gradient carried along
    la::BwdParams b;
    std::memset(&b, 0, sizeof b);
    b.q = q;
    b.k = k;
    b.v = v;
    b.dout = dout;
    b.log_alpha = p.log_alpha;
    b.st_fwd = states ? states : static_cast<const void*>(ws + w.fwd);
    b.g_entry = pl.P > 1 ? p.ws_S : dS_final;
    b.dS0 = dS0;
    b.dq = dq;
    b.dk = dk;
    b.dv = dv;
    b.dlog_alpha = dlog_alpha;
    b.L = d->L;
    b.H = d->H;
    b.BH = BH;
    b.nchunks = pl.nchunks;
    b.P = pl.P;
    b.cps = pl.cps;
    b.phi_elu1 = p.phi_elu1;
    std::memcpy(b.log2_gamma, p.log2_gamma, sizeof b.log2_gamma);
    e = timed_launch(la::K_BWD, s, [&] { return bwd_launch(d, b, gate_mode, s); });
    if (e != hipSuccess) return hip_fail(e, "backward launch");
    return LA_OK;
}

int la_delta_chunk(const la_desc* d) {
    if (check_desc(d) != LA_OK) return 0;
    return (d->dtype != LA_BF16 && d->dk >= 128) ? 32 : 64;
}

la_status la_delta_fwd(const la_desc* d, const void* q, const void* k, const void* v,
                       const float* beta, const float* S0, void* out, float* S_final,
                       void* stream) {
    g_errmsg[0] = '\0';
    const la_status st = check_delta(d);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !beta || !out)
        return fail(LA_ERR_INVALID, "q, k, v, beta and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(out) ||
        (S0 && !aligned16(S0)) || (S_final && !aligned16(S_final)))
        return fail(LA_ERR_INVALID, "device pointers must be 16-byte aligned");
    la::DeltaParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.k = k;
    p.v = v;
    p.beta = beta;
    p.S0 = S0;
    p.out = out;
    p.S_final = S_final;
    p.L = d->L;
    p.H = d->H;
    p.BH = d->B * d->H;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = timed_launch(la::K_DELTA, s, [&] { return delta_launch(d, p, false, s); });
    if (e != hipSuccess) return hip_fail(e, "delta prefill launch");
    return LA_OK;
}

la_status la_delta_decode_step(const la_desc* d, const void* q, const void* k, const void* v,
                               const float* beta, float* S, void* out, void* stream) {
    g_errmsg[0] = '\0';
    const la_status st = check_delta(d);
    if (st != LA_OK) return st;
    if (d->L != 1) return fail(LA_ERR_INVALID, "decode needs L == 1 (L=%d)", d->L);
    if (!q || !k || !v || !beta || !S || !out)
        return fail(LA_ERR_INVALID, "q, k, v, beta, S and out must be non-NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(beta) || !aligned16(S) ||
        !aligned16(out))
        return fail(LA_ERR_INVALID, "device pointers must be 16-byte aligned");
    la::DeltaParams p;
    std::memset(&p, 0, sizeof p);
    p.q = q;
    p.k = k;
    p.v = v;
    p.beta = beta;
    p.S = S;
    p.out = out;
    p.L = 1;
    p.H = d->H;
    p.BH = d->B * d->H;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = timed_launch(la::K_DELTA_DECODE, s, [&] { return delta_launch(d, p, true, s); });
    if (e != hipSuccess) return hip_fail(e, "delta decode launch");
    return LA_OK;
}

la_status la_decode_step(const la_desc* d, const void* q, const void* k, const void* v,
                         int gate_mode, const float* gate, float* S, float* z, void* out,
                         void* stream) {
    g_errmsg[0] = '\0';
    la_status st = check_desc(d, false, true);
    if (st != LA_OK) return st;
    if (d->L != 1) return fail(LA_ERR_INVALID, "decode needs L == 1 (L=%d)", d->L);
    if (!q || !k || !v || !out || !S) return fail(LA_ERR_INVALID, "q, k, v, S and out must be non-NULL");
    if (d->normalize && !z) return fail(LA_ERR_INVALID, "normalize needs z");
    if (!d->normalize && z) return fail(LA_ERR_INVALID, "z given without normalize");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(S) ||
        (z && !aligned16(z)))
        return fail(LA_ERR_INVALID, "device pointers must be 16-byte aligned");
    la::DecodeParams p;
    std::memset(&p, 0, sizeof p);
    st = check_gate(d, gate_mode, gate, true, nullptr, p.gamma);
    if (st != LA_OK) return st;
    p.q = q;
    p.k = k;
    p.v = v;
    p.log_alpha = device_gate(gate_mode) ? gate : nullptr;
    p.S = S;
    p.z = z;
    p.out = out;
    p.H = d->H;
    p.BH = d->B * d->H;
    p.phi_elu1 = d->phi == LA_PHI_ELU1;
    p.normalize = d->normalize;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = timed_launch(la::K_DECODE, s, [&] {
        return la::launch_decode(p, d->dk, d->dv, d->dtype == LA_BF16, gate_mode, s);
    });
    if (e != hipSuccess) return hip_fail(e, "decode launch");
    return LA_OK;
}

la_status la_profile_begin(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (auto& r : g_prof) {
        g_event_pool.push_back(r.a);
        g_event_pool.push_back(r.b);
    }
    g_prof.clear();
    g_prof_on = true;
    return LA_OK;
}

la_status la_profile_end(void) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_on = false;
    return LA_OK;
}

la_status la_profile_query(const char* kernel, int* launches, double* total_ms) {
    if (!kernel || !launches || !total_ms) return fail(LA_ERR_INVALID, "NULL argument");
    int id = -1;
    for (int i = 0; i < la::K_COUNT; ++i)
        if (std::strcmp(kernel, kKernelNames[i]) == 0) id = i;
    if (id < 0) return fail(LA_ERR_INVALID, "unknown kernel family '%s'", kernel);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    int n = 0;
    double ms = 0.0;
    for (auto& r : g_prof) {
        if (r.kernel != id) continue;
        hipError_t e = hipEventSynchronize(r.b);
        if (e != hipSuccess) return hip_fail(e, "event synchronize");
        float x = 0.f;
        e = hipEventElapsedTime(&x, r.a, r.b);
        if (e != hipSuccess) return hip_fail(e, "event elapsed time");
        ms += x;
        ++n;
    }
    *launches = n;
    *total_ms = ms;
    return LA_OK;
}

}  // extern "C"
