// chunk_kernel.h -- chunkwise-parallel prefill of the unified recurrence on
// gfx950 matrix cores.
//
// Form computed ("Module 22: Linear & Recurrent Attention", section "The
// Three Faces of Retention", generalised to a diagonal per-channel gate as in
// the gate table of "The One Recurrence Behind Them All"; ragged last chunk
// as in linear_attn_chunkwise of "linear_sparse_attention.py").  For a chunk
// of c tokens with chunk-local t, s and b_t = sum_{r<=t} log a_r (per key
// channel, inclusive):
//
//   o_t   = (phi(q_t) * e^{b_t})^T S_prev
//         + sum_{s<=t} [sum_i phi(q_ti) phi(k_si) e^{b_ti - b_si}] v_s
//   S_new = diag(e^{b_{c-1}}) S_prev + sum_s (phi(k_s) * e^{b_{c-1} - b_s}) v_s^T
//
// Matrix-core mapping per chunk (C tokens, d_k x d_v state, fp32 accum).
// The score and output products are computed transposed so that every lane
// ends up holding four consecutive s (or output columns) and writes them as
// one packed run:
//   op1  P^T = Kh Qh^T                [C x C], lower-triangular 16x16 tiles
//   op2  O^T = S'^T Qh^T + V^T P^T    [d_v x C]
//   op3  S'' = Kt^T V                 [d_k x d_v], onto the scaled state
// Decay placement by gate mode:
//   NONE  : no scaling.
//   GAMMA : P masked by gamma^(t-s) elementwise (exact for gamma = 0); the
//           S'^T Qh^T term scaled per token by gamma^(t+1); Kt by
//           gamma^(c-1-s); the state by gamma^c.  All factors <= 1.
//   DIAG  : factorised around a reference r = b at the chunk middle:
//           Qh = q e^{b_t - r}, Kh = Kt = k e^{r - b_s}; the state rows are
//           scaled by e^{r} before use and by e^{b_{c-1} - r} after the
//           update, so S_new = e^{b_{c-1}-r} (e^{r} S + Kh^T V).  The
//           after-factor of one chunk and the before-factor of the next are
//           applied as one product.
// The state S stays in fp32 matrix-core accumulators for the whole segment;
// wave w owns state columns [w*WN, (w+1)*WN).  For the S'^T Qh^T product the
// accumulators are converted in registers into A operands: lane (n, g) holds
// state rows 16m + 4g + i of column n, so Qh is stored with its d_k index
// permuted within every 32 channels such that one 16-byte read returns the
// matching rows (Kh uses the same layout, which leaves Kh Qh^T unchanged).
//
// LDS tiles are unpadded and XOR-swizzled in 16-byte units so that both the
// fragment reads (16 consecutive rows, one unit) and the transposed tile
// writes (rows two apart) spread over the banks.
//
// Global memory is read through buffer descriptors covering one (b,h) slice:
// tokens past L read as zeros and output rows past L are dropped by the
// hardware range check, so the ragged tail needs no branches.
//
// One workgroup runs one (b,h) segment of consecutive chunks.  SONLY = true
// is the state pass: the same loop without q, P and outputs, started from a
// zero state, writing the segment's end state, its decay product and its
// normaliser part to the workspace.
//
// Two more state-only variants serve the backward pass:
//  * STORE starts each segment from its entry state (after the segment
//    scan) and writes the true state at every chunk boundary (also on the
//    main pass, for a forward that keeps its states for the backward);
//  * REV aggregates the recurrence of the state gradient over a segment,
//    G_prev = A_c G + sum_t (phi(q_t) * e^{b_t}) do_t^T, which is the state
//    update with k -> phi(q), v -> do, the key factor replaced by the query
//    factor, the before/after factors swapped, and the chunks taken in
//    reverse order (the caller passes q and do in the k and v slots); the
//    gradient kernel carries G through each segment itself.
#pragma once

#include <type_traits>

#include "la_device.h"
#include "la_internal.h"

namespace la {

// Channels per thread in the global -> register mapping: 4 where the chunk
// still leaves every thread an even run of tokens, else 2.
constexpr int run_width(int D, int NT, int C) {
    return (NT % (D / 4) == 0 && NT / (D / 4) >= 2 && C % (NT / (D / 4)) == 0 &&
            (C / (NT / (D / 4))) % 2 == 0) ? 4 : 2;
}

template <int DK_, int DV_, int C_, bool BF16_, int GATE_, bool SONLY_, int NW_>
struct ChunkCfg {
    static constexpr int DK = DK_, DV = DV_, C = C_, GATE = GATE_, NW = NW_;
    static constexpr bool BF16 = BF16_, SONLY = SONLY_;
    using T = Elem<BF16>;
    using E = typename T::E;
    using Pair = typename T::Pair;
    using Frag = typename T::Frag;
    static constexpr int NT = 64 * NW;                 // threads
    static constexpr int WN = DV / NW;                 // state columns per wave
    static constexpr int NB = WN / 16;                 // 16-column blocks per wave
    static constexpr int MB = DK / 16;                 // 16-row blocks of the state
    static constexpr int TB = C / 16;                  // 16-row blocks of a chunk
    static constexpr int KPL = T::KPL, MK = T::MK;
    static constexpr int CP = C < MK ? MK : C;         // token extent of s-contractions
    static constexpr int UE = 16 / (int)sizeof(E);     // elements per 16-byte unit
    static constexpr int QU = DK / UE;                 // units per q/k row
    static constexpr int TU = CP / UE;                 // units per transposed row / P row
    // q/k tiles swizzle over up to 16 units (256 bytes): the LDS has 64
    // four-byte banks, so 16 consecutive rows of a fragment read fall on 16
    // different bank groups
    static constexpr int QMASK = (QU < 16 ? QU : 16) - 1;
    static constexpr int TMASK = (TU < 8 ? TU : 8) - 1;
    // global -> register mapping: each thread owns a run of CW adjacent key
    // channels (VW value channels) over KTPG (VTPG) consecutive tokens and
    // reads it with one buffer load per token
    static constexpr int CW = run_width(DK, NT, C), VW = run_width(DV, NT, C);
    static constexpr int KCP = DK / CW, KTG = NT / KCP, KTPG = C / KTG;
    static constexpr int VCP = DV / VW, VTG = NT / VCP, VTPG = C / VTG;
    static constexpr int KWORDS = CW * (int)sizeof(E) / 4;   // 32-bit words per run
    static constexpr int VWORDS = VW * (int)sizeof(E) / 4;
    // chunks of k, v and gates held in registers ahead of use.  One chunk of
    // main-pass work covers the memory latency, and a second register set
    // would only take registers from the rest of its loop; the state pass
    // has a shorter chunk and registers to spare, so it keeps two (bf16)
    static constexpr int PD = (SONLY && BF16) ? 2 : 1;
    // fp32 main passes at d = 128 hold 64 registers per chunk of k, v, q and
    // gates; prefetched a chunk ahead they stay live through every phase
    // and the kernel spills heavily, so those load each chunk as its step
    // begins instead
    static constexpr bool PREFETCH = BF16 || SONLY || DK < 128;
    // main pass under a vector gate (DIAG, SCALAR): chunks whose gates are
    // too strong for the chunk-middle reference take the sub-chunk path
    static constexpr bool VGM = (GATE == LA_GATE_DIAG || GATE == LA_GATE_SCALAR) && !SONLY;
    static constexpr int TPW = C / NW;                // tokens per wave (consecutive)
    // the chunk-middle factors stay below 2^LIM while each half chunk's
    // log2-gate sum does; a wave votes for the sub-chunk path when a
    // channel's sum over its tokens is below LIM / (waves per half)
    static constexpr float LIM = 120.f;
    static constexpr float WAVE_THR = -LIM / (NW >= 2 ? NW / 2 : 1);
    static_assert(DV % (16 * NW) == 0 && DK % 16 == 0 && C % 16 == 0, "tile shape");
    static_assert(!BF16 || DK % 32 == 0, "bf16 needs d_k >= 32");
    static_assert(NT % KCP == 0 && NT % VCP == 0, "channel-run mapping");
    static_assert((KTPG * (int)sizeof(E) <= 16 || KTPG * (int)sizeof(E) % 16 == 0) &&
                  (VTPG * (int)sizeof(E) <= 16 || VTPG * (int)sizeof(E) % 16 == 0),
                  "a transposed run stays within one 16-byte unit or is whole units");
    static_assert(KTG >= 2 && KTG % 2 == 0 && KTPG >= 1 && VTPG >= 1, "token groups");
    static_assert(KTG * KTPG == C && VTG * VTPG == C, "token groups cover the chunk");
    static_assert(8 % KTPG == 0 && C % NW == 0,
                  "a thread's run stays in one 16-token block, ending at or before its eighth token");
};

template <class Cfg>
struct ChunkSmem {
    using E = typename Cfg::E;
    static constexpr int CQ = Cfg::SONLY ? 1 : Cfg::C;
    // the scalar-gate passes without outputs keep two sets of the per-chunk
    // tiles and factors (chunk parity), so that a chunk's tiles are filled
    // while the previous chunk's state products still read theirs, with no
    // barrier between: 75 -> 66 us for the state pass of the 32768-token,
    // 16-head scalar-gate workload.  The same for the diagonal-gate and
    // gamma state passes measured 2% slower, so those keep one set.
    static constexpr int NBUF = (Cfg::SONLY && Cfg::GATE == LA_GATE_SCALAR) ? 2 : 1;
    alignas(16) E q[CQ][Cfg::DK];        // Qh, [t][permuted, swizzled i]
    alignas(16) E k[CQ][Cfg::DK];        // Kh, [s][permuted, swizzled i]
    alignas(16) E kt[NBUF][Cfg::DK][Cfg::CP];  // Kt, [i][swizzled s]
    alignas(16) E vt[NBUF][Cfg::DV][Cfg::CP];  // V^T, [n][swizzled s]
    alignas(16) E p[CQ][Cfg::CP];        // masked scores, [t][swizzled s]
    // per-wave log2-gate sums (a2), and the group norm's per-wave token sums
    // (store phase of the main pass): live between different barriers
    // vector gates, main pass, sub-chunk path: per 16-token block the
    // in-wave prefix at its eighth and at its last token (the wave prefix is
    // added on use), the state factors around its state term and the
    // normaliser entering it; one vote per wave
    static constexpr int TBV = Cfg::VGM ? Cfg::TB : 1;
    static constexpr int DKV = Cfg::VGM ? Cfg::DK : 1;
    // also the sub-chunk normaliser (after op1, before the store phase)
    union {
        alignas(16) float tot[NBUF][Cfg::NW][Cfg::DK];
        float2 gnp[Cfg::SONLY ? 1 : Cfg::NW][Cfg::SONLY ? 1 : Cfg::C];
        float zs[TBV][DKV];
    };
    alignas(16) float bmid[TBV][DKV];
    alignas(16) float bend[TBV][DKV];
    alignas(16) float sa[TBV][DKV];
    alignas(16) float sb[TBV][DKV];
    int wslow[Cfg::VGM ? Cfg::NW : 1];
    alignas(16) float scale[NBUF][Cfg::DK];    // per-row state factor applied this chunk
    alignas(16) float pre[NBUF][Cfg::DK];      // this chunk's before/after factors
    alignas(16) float post[NBUF][Cfg::DK];
    alignas(16) float segsum[Cfg::DK];   // DIAG: summed log2-gates of this segment
    float gpow[Cfg::C + 2];              // gamma^j
    float z[Cfg::DK];
    float den[Cfg::C];
};

// Position of logical channel l in row `row` of a q/k tile.  bf16 tiles
// store, within every 32 channels, the channels 4g..4g+3 next to
// 16+4g..16+4g+3 (the order in which the state accumulators hand out their
// rows), then swizzle 16-byte units by the row.
template <class Cfg>
__device__ __forceinline__ int qk_pos(int row, int l) {
    int p = l;
    if constexpr (Cfg::BF16) p = (l & ~31) + 8 * ((l & 15) >> 2) + 4 * ((l & 31) >> 4) + (l & 3);
    const int u = p / Cfg::UE, e = p % Cfg::UE;
    return ((u ^ (row & Cfg::QMASK)) * Cfg::UE) + e;
}
// Position of the physical k-slot run that starts at permuted position pp
// (a multiple of the unit, or of the slot count for fp32) in row `row`.
template <class Cfg>
__device__ __forceinline__ int qk_phys(int row, int pp) {
    const int u = pp / Cfg::UE, e = pp % Cfg::UE;
    return ((u ^ (row & Cfg::QMASK)) * Cfg::UE) + e;
}
// Position of token s in row `row` of a transposed tile (kt, vt).  With
// 128-byte rows (bf16, 64-token chunks) the units are XOR-swizzled by
// row ^ (row >> 2): the 16-row fragment reads of the state update and of
// the value operands then run without bank conflicts, where row ^ (row >> 3)
// left every one of them two-way conflicted (measured per access pattern on
// gfx950; the 8-byte stores that fill the tile are two-way under every XOR
// swizzle tried).
template <class Cfg>
__device__ __forceinline__ int tr_pos(int row, int s) {
    constexpr int SH = Cfg::CP * (int)sizeof(typename Cfg::E) == 128 ? 2 : 3;
    const int u = s / Cfg::UE, e = s % Cfg::UE;
    return ((u ^ ((row ^ (row >> SH)) & Cfg::TMASK)) * Cfg::UE) + e;
}
// Position of token s in row t of the score tile.
template <class Cfg>
__device__ __forceinline__ int p_pos(int t, int s) {
    const int u = s / Cfg::UE, e = s % Cfg::UE;
    return ((u ^ (t & Cfg::TMASK)) * Cfg::UE) + e;
}

// Store a run of N consecutive tokens (starting at s0, a multiple of N) of
// one transposed-tile row, held as N/2 packed token pairs, one 16-byte unit
// (or less) per vector write.
template <class Cfg, int N>
__device__ __forceinline__ void store_pairs(typename Cfg::E* rowp, int row, int s0,
                                            const typename Cfg::Pair* w) {
    using E = typename Cfg::E;
    constexpr int PIECE = N < Cfg::UE ? N : Cfg::UE;      // elements per write
    constexpr int BYTES = PIECE * (int)sizeof(E);
    using V = typename std::conditional<
        BYTES == 16, uint4, typename std::conditional<BYTES == 8, uint2, uint32_t>::type>::type;
    constexpr int PP = PIECE / 2;                          // pairs per write
#pragma unroll
    for (int q = 0; q < N / PIECE; ++q) {
        V v;
        __builtin_memcpy(&v, w + q * PP, sizeof v);
        *reinterpret_cast<V*>(rowp + tr_pos<Cfg>(row, s0 + q * PIECE)) = v;
    }
}
// Channel c of two runs at consecutive tokens as one token pair.
template <class Cfg, int N>
__device__ __forceinline__ typename Cfg::Pair token_pair(const Words<N>& a, const Words<N>& b, int c) {
    if constexpr (Cfg::BF16)
        return __builtin_amdgcn_perm(b.w[c >> 1], a.w[c >> 1], (c & 1) ? 0x07060302u : 0x05040100u);
    else
        return make_float2(__uint_as_float(a.w[c]), __uint_as_float(b.w[c]));
}

template <class Cfg>
__device__ __forceinline__ void scale_rows(f32x4_t (&acc)[Cfg::MB][Cfg::NB], const float* f, int g) {
#pragma unroll
    for (int mb = 0; mb < Cfg::MB; ++mb) {
        const f32x4_t s = *reinterpret_cast<const f32x4_t*>(&f[16 * mb + 4 * g]);
#pragma unroll
        for (int nb = 0; nb < Cfg::NB; ++nb) acc[mb][nb] *= s;
    }
}

// 4x4 transpose within each quad of lanes: on entry lane q of a quad holds
// x[j] = M[j][q], on exit x[j] = M[q][j].  Two butterfly exchanges (lanes
// q ^ 1, then q ^ 2), each moving two of the four values.
__device__ __forceinline__ void quad_transpose(float (&x)[4], int q) {
    {
        const bool odd = q & 1;
        const float a = odd ? x[0] : x[1], b = odd ? x[2] : x[3];
        const float a2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false));
        const float b2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b), 0xB1, 0xF, 0xF, false));
        if (odd) { x[0] = a2; x[2] = b2; } else { x[1] = a2; x[3] = b2; }
    }
    {
        const bool hi = q & 2;
        const float a = hi ? x[0] : x[2], b = hi ? x[1] : x[3];
        const float a2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false));
        const float b2 = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(b), 0x4E, 0xF, 0xF, false));
        if (hi) { x[0] = a2; x[1] = b2; } else { x[2] = a2; x[3] = b2; }
    }
}

// 12 wait states: more than any matrix-core result needs (10 for the fp32
// operation) before another instruction may touch its registers.  The
// compiler pads straight-line code itself; after a matrix product that a
// branch can follow, the kernels pad explicitly, since padding has been seen
// to go missing across such branches.  The scheduling barriers keep the
// compiler from moving matrix products (register-only instructions) past
// the padding.
__device__ __forceinline__ void mfma_drain() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 3" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

template <class Cfg, bool ELU1, bool REV = false, bool STORE = false, bool EPI = false, bool ROB = false>
__global__ __launch_bounds__(Cfg::NT) void chunk_kernel(const ChunkParams p) {
    constexpr int DK = Cfg::DK, DV = Cfg::DV, C = Cfg::C, GATE = Cfg::GATE;
    constexpr int NB = Cfg::NB, MB = Cfg::MB, TB = Cfg::TB, NW = Cfg::NW;
    constexpr int KPL = Cfg::KPL, MK = Cfg::MK, CP = Cfg::CP;
    constexpr int KCP = Cfg::KCP, KTG = Cfg::KTG, KTPG = Cfg::KTPG, CW = Cfg::CW;
    constexpr int VCP = Cfg::VCP, VTPG = Cfg::VTPG, VW = Cfg::VW;
    constexpr bool SONLY = Cfg::SONLY, BF16 = Cfg::BF16;
    constexpr int NBUF = ChunkSmem<Cfg>::NBUF;
    constexpr int ES = (int)sizeof(typename Cfg::E);
    // lanes that share one normaliser row (NRL) or one z channel (NCL): the
    // workgroup's threads over the rows or channels, 1 to 16
    constexpr int NRL = Cfg::NT / C >= 16 ? 16 : (Cfg::NT / C < 1 ? 1 : Cfg::NT / C);
    constexpr int NCL = Cfg::NT / DK >= 16 ? 16 : (Cfg::NT / DK < 1 ? 1 : Cfg::NT / DK);
    // unroll of the normaliser's sums: whole, or by four where the whole
    // unroll spills registers (d = 128; fp32 at d = 32 in the 128-token tile)
    constexpr int NUNR = (DK >= 128 || (!BF16 && DK == 32 && C >= 128)) ? 4 : 32;
    using T = typename Cfg::T;
    using E = typename Cfg::E;
    using Pair = typename Cfg::Pair;
    using Frag = typename Cfg::Frag;
    // the diagonal and the per-token scalar gate share one path (a scalar
    // gate is a diagonal one with equal channels)
    constexpr bool VG = GATE == LA_GATE_DIAG || GATE == LA_GATE_SCALAR;

    __shared__ ChunkSmem<Cfg> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int r = lane & 15, g = lane >> 4;
    const int P = p.P;
    static_assert(SONLY || !REV, "the reversed walk is state-only");
    static_assert(!(REV && STORE), "the reversed walk only aggregates segments");
    static_assert(!(STORE && EPI), "no epilogue with the boundary states");
    static_assert(!(SONLY && EPI), "the output epilogue belongs to the main pass");
    // the aggregate pass skips the segment it would end with (the last one,
    // or the first one when reversed)
    constexpr bool AGG = SONLY && !STORE;
    // cache policy of the q, k, v and gate loads: non-temporal streams in
    // the aggregate and main passes; the default in the passes that store
    // every boundary state, whose inputs the gradient kernel reads next
    constexpr int LAUX = STORE ? 0 : LOAD_NT;
    // the forward aggregate pass walks its segment from the last chunk to
    // the first (see cof below)
    constexpr bool BACKAGG = AGG && !REV;
    const int PS = AGG ? P - 1 : P;
    const int seg = blockIdx.x % PS + ((AGG && REV) ? 1 : 0);
    // packed sequences run in the given order (longest first), the heads of
    // one sequence side by side
    int bh = blockIdx.x / PS;
    if (p.seq_order) {
        const int nseq = p.BH / p.H;
        bh = min(max(p.seq_order[bh / p.H], 0), nseq - 1) * p.H + bh % p.H;
    }
    const int h = bh % p.H;
    // the token range of this (b,h) slice: all L tokens of slice bh, or
    // (packed sequences) tokens [cu[n], cu[n+1]) of head h's p.L tokens,
    // clamped to that head's range
    int L = p.L;
    size_t rows0 = (size_t)bh * L;
    if (p.cu_seqlens) {
        const int n = bh / p.H;
        const int s0 = min(max(p.cu_seqlens[n], 0), p.L);
        const int s1 = min(max(p.cu_seqlens[n + 1], s0), p.L);
        L = s1 - s0;
        rows0 = (size_t)h * p.L + s0;
    }
    // the chunk length: the tile C, or a multiple of 16 below it (the rest
    // of the tile then holds no tokens: its gates and keys are masked and
    // its output rows dropped)
    const int CR = C > 16 ? p.chunk : C;
    const int nchunks = (L + CR - 1) / CR;
    const int c_begin = seg * p.cps;
    const int c_end = min(c_begin + p.cps, nchunks);
    const bool norm = p.normalize != 0;
    // vector gates, main pass: the kernel without the sub-chunk path (ROB
    // false) hands a segment with a chunk too strong for the chunk-middle
    // reference to the one with it (ROB true), which runs only such segments
    static_assert(!ROB || Cfg::VGM, "the sub-chunk kernel is a vector-gate main pass");
    constexpr bool SUB = Cfg::VGM && ROB;
    int* const seg_flag = Cfg::VGM ? p.slow_flags + ((size_t)bh * P + seg) : nullptr;
    if constexpr (ROB) {
        if (__builtin_amdgcn_readfirstlane(*seg_flag) == 0) return;
    }

    const int kcp = tid % KCP, ktg = tid / KCP;
    const int vcp = tid % VCP, vtg = tid / VCP;
    const int colbase = wave * Cfg::WN;

    // ---- buffer descriptors over this (b,h) slice
    const __amdgpu_buffer_rsrc_t rq =
        make_rsrc(reinterpret_cast<const E*>(p.q) + rows0 * DK, (uint32_t)L * DK * ES);
    const __amdgpu_buffer_rsrc_t rk =
        make_rsrc(reinterpret_cast<const E*>(p.k) + rows0 * DK, (uint32_t)L * DK * ES);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(reinterpret_cast<const E*>(p.v) + rows0 * DV, (uint32_t)L * DV * ES);
    // log-gates: DIAG one per token and key channel, SCALAR one per token
    const __amdgpu_buffer_rsrc_t rla =
        make_rsrc(GATE == LA_GATE_DIAG ? (const void*)(p.log_alpha + rows0 * DK)
                  : GATE == LA_GATE_SCALAR ? (const void*)(p.log_alpha + rows0) : p.q,
                  GATE == LA_GATE_DIAG ? (uint32_t)L * DK * 4
                  : GATE == LA_GATE_SCALAR ? (uint32_t)L * 4 : 0u);
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(SONLY ? p.q : (const void*)(reinterpret_cast<const E*>(p.out) + rows0 * DV),
                  SONLY ? 0u : (uint32_t)L * DV * ES);

    // ---- one-time LDS set-up: zero the tiles whose padding is read as zeros
    {
        if constexpr (CP > C) {
            E* z0p = &sm.kt[0][0][0];
            for (int i = tid; i < NBUF * DK * CP; i += Cfg::NT) z0p[i] = E(0);
            E* z1p = &sm.vt[0][0][0];
            for (int i = tid; i < NBUF * DV * CP; i += Cfg::NT) z1p[i] = E(0);
        }
        if constexpr (!SONLY) {
            E* z2p = &sm.p[0][0];
            for (int i = tid; i < C * CP; i += Cfg::NT) z2p[i] = E(0);
        }
        if constexpr (!SONLY) {
            // without the normaliser every row divides by one, so the output
            // epilogue has no branch: a uniform branch between the last
            // matrix-core write of the accumulators and their first VALU read
            // has been seen to lose the wait states that read needs
            if (!norm)
                for (int j = tid; j < C; j += Cfg::NT) sm.den[j] = 1.0f;
        }
        if constexpr (GATE == LA_GATE_GAMMA) {
            const float l2g = p.log2_gamma[h];
            for (int j = tid; j < C + 2; j += Cfg::NT) sm.gpow[j] = j == 0 ? 1.0f : exp2f((float)j * l2g);
        }
    }

    // ---- initial state
    const size_t SS = (size_t)DK * DV;
    const float* Sin = nullptr;
    const float* zin = nullptr;
    if constexpr (!AGG) {
        if (P > 1) {
            Sin = p.ws_S + ((size_t)bh * P + seg) * SS;
            zin = p.ws_z + ((size_t)bh * P + seg) * DK;
        } else {
            Sin = p.S0 ? p.S0 + (size_t)bh * SS : nullptr;
            zin = p.z0 ? p.z0 + (size_t)bh * DK : nullptr;
        }
    }
    f32x4_t accS[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                accS[mb][nb][i] = Sin ? Sin[(size_t)(16 * mb + 4 * g + i) * DV + colbase + 16 * nb + r] : 0.0f;
    if (norm && tid < DK) sm.z[tid] = zin ? zin[tid] : 0.0f;

    // segment bookkeeping of the ktg == 0 threads lives in LDS: the previous
    // chunk's after-factor (post) and the segment's summed log2-gates
    if (tid < DK) {
#pragma unroll
        for (int b = 0; b < NBUF; ++b) sm.post[b][tid] = 1.0f;
        sm.segsum[tid] = 0.0f;
    }
    float seg_g = 1.0f;                  // GAMMA: product of gamma^c

    // ---- register prefetch, two chunks ahead (byte offsets within the slice)
    // k, v and the gates run PD chunks ahead (PD register sets); q, needed
    // only by the main pass, one chunk ahead
    struct ChunkRegs {
        Words<Cfg::KWORDS> k[KTPG];
        Words<Cfg::VWORDS> v[VTPG];
        Words<CW> la[VG ? KTPG : 1];
    };
    Words<Cfg::KWORDS> qreg[SONLY ? 1 : KTPG];
    // output epilogue (group norm over each token's d_v outputs, then times
    // swish of the gate): the gate runs of this lane's outputs, one chunk
    // ahead, and the norm's per-channel scale and shift
    constexpr int OW = 4 * ES / 4;   // words of a 4-channel output run
    Words<OW> greg[EPI ? NB : 1][EPI ? TB : 1];
    float gnw[EPI ? NB : 1][4], gnb[EPI ? NB : 1][4];
    const __amdgpu_buffer_rsrc_t rgate =
        make_rsrc(EPI && p.gn_gate ? (const void*)(reinterpret_cast<const E*>(p.gn_gate) + rows0 * DV) : p.q,
                  EPI && p.gn_gate ? (uint32_t)L * DV * ES : 0u);
    if constexpr (EPI) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int n = colbase + 16 * nb + 4 * g + i;
                gnw[nb][i] = p.gn_w ? p.gn_w[(size_t)h * DV + n] : 1.0f;
                gnb[nb][i] = p.gn_b ? p.gn_b[(size_t)h * DV + n] : 0.0f;
            }
    }
    auto load_chunk = [&](int c, ChunkRegs& rg) {
        const uint32_t t0 = (uint32_t)c * CR;
        const uint32_t okk = ((t0 + ktg * KTPG) * DK + CW * kcp) * ES;
        const uint32_t ovv = ((t0 + vtg * VTPG) * DV + VW * vcp) * ES;
        const uint32_t oaa = ((t0 + ktg * KTPG) * DK + CW * kcp) * 4;
#pragma unroll
        for (int j = 0; j < KTPG; ++j) {
            rg.k[j] = buf_load_words<Cfg::KWORDS, LAUX>(rk, okk + j * DK * ES);
            if constexpr (GATE == LA_GATE_DIAG) rg.la[j] = buf_load_words<CW, LAUX>(rla, oaa + j * DK * 4);
            if constexpr (GATE == LA_GATE_SCALAR) {
                // one gate per token, the same for every channel of the run
                const uint32_t w =
                    __builtin_amdgcn_raw_buffer_load_b32(rla, (t0 + ktg * KTPG + j) * 4, 0, LAUX);
#pragma unroll
                for (int i = 0; i < CW; ++i) rg.la[j].w[i] = w;
            }
        }
#pragma unroll
        for (int j = 0; j < VTPG; ++j) rg.v[j] = buf_load_words<Cfg::VWORDS, LAUX>(rv, ovv + j * DV * ES);
    };
    auto load_q = [&](int c) {
        if constexpr (!SONLY) {
            const uint32_t okk = (((uint32_t)c * CR + ktg * KTPG) * DK + CW * kcp) * ES;
#pragma unroll
            for (int j = 0; j < KTPG; ++j) qreg[j] = buf_load_words<Cfg::KWORDS, LAUX>(rq, okk + j * DK * ES);
        }
    };
    // the gate runs of chunk c's outputs (loaded after the previous chunk's
    // outputs are stored; without a gate tensor the descriptor is empty)
    auto load_gate = [&](int c) {
        if constexpr (EPI) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const uint32_t og = (((uint32_t)c * CR + 16 * tb + r) * DV + colbase + 16 * nb + 4 * g) * ES;
                    greg[nb][tb] = buf_load_words<OW>(rgate, og);
                }
        }
    };
    constexpr float kLog2e = 1.4426950408889634f;

    // chunk handled at iteration ci: reverse order for the gradient pass,
    // and for the forward aggregate pass, whose result does not depend on
    // the order (each chunk's K^T V is weighted by the decay of the chunks
    // after it, accumulated as the walk goes) and whose last reads -- the
    // segment's first chunks -- are then the most recently used data when
    // the main pass starts there
    auto cof = [&](int ci) { return (REV || BACKAGG) ? c_begin + c_end - 1 - ci : ci; };
    // backward walk: log2 decay of the chunks already walked, per owned
    // channel (vector gates) or as a product (gamma)
    float eacc[CW];
#pragma unroll
    for (int i = 0; i < CW; ++i) eacc[i] = 0.f;
    // the true state in the accumulators, into boundary slot `slot` in the
    // element type: rows times the after-factor still pending (diagonal
    // gate), then a 4x4 transpose within each lane quad so that every lane
    // writes four consecutive columns of one row
    auto store_state = [&](int slot, int bsel) {
        E* rows = reinterpret_cast<E*>(p.st_rows) + ((size_t)bh * p.st_slots + slot) * SS;
        const int q4 = lane & 3;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            f32x4_t f = {1.f, 1.f, 1.f, 1.f};
            if constexpr (VG) f = *reinterpret_cast<const f32x4_t*>(&sm.post[bsel][16 * mb + 4 * g]);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float x[4] = {accS[mb][nb][0] * f[0], accS[mb][nb][1] * f[1],
                              accS[mb][nb][2] * f[2], accS[mb][nb][3] * f[3]};
                quad_transpose(x, q4);
                E* dst = rows + (size_t)(16 * mb + 4 * g + q4) * DV + colbase + 16 * nb + (r & ~3);
                store_run<BF16, 4>(dst, x);
            }
        }
    };

    // one chunk (iteration ci): consumes rg, then refills it with the chunk
    // PD iterations ahead
    auto step = [&](const int ci, ChunkRegs& rg) -> bool {
        const int c = cof(ci);
        const int bsel = NBUF > 1 ? (ci & 1) : 0;   // this chunk's tile and factor set
        const int t0 = c * CR;
        const int clen = min(CR, L - t0);
        if constexpr (!Cfg::PREFETCH) {
            load_q(c);
            load_chunk(c, rg);
        }
        // a chunk shorter than the tile: the tile's later tokens are the next
        // chunk's, so their gates count as zero and their output rows fall
        // outside the store descriptor's range (tokens past L read as zeros
        // by themselves)
        if constexpr (VG && C > 16) {
            if (CR < C) {
#pragma unroll
                for (int j = 0; j < KTPG; ++j)
                    if (ktg * KTPG + j >= clen) {
#pragma unroll
                        for (int i = 0; i < CW; ++i) rg.la[j].w[i] = 0u;
                    }
            }
        }
        const __amdgpu_buffer_rsrc_t roc =
            (C > 16 && CR < C) ? make_rsrc(SONLY ? p.q : (const void*)(reinterpret_cast<const E*>(p.out) + rows0 * DV),
                                           SONLY ? 0u : (uint32_t)(t0 + clen) * DV * ES)
                               : ro;

        // ---- a2: chunk-local log2-gate sums.  Each thread sums its own run;
        // the token groups of one wave (lanes KCP apart hold the same channels
        // at consecutive groups) are combined by a scan over lane shuffles,
        // and only the wave totals go through LDS.
        float gexc[CW], gmid[CW];   // earlier groups of this wave; one wave: chunk middle
#pragma unroll
        for (int i = 0; i < CW; ++i) gexc[i] = gmid[i] = 0.f;
        if constexpr (VG) {
            // a scalar gate is the same in every channel: its sums are formed
            // once (channel 0) and repeated, so that everything computed from
            // them below is one value per token
            constexpr int GC = GATE == LA_GATE_SCALAR ? 1 : CW;
            float gsum[CW], incl[CW], wsum[CW];
#pragma unroll
            for (int i = 0; i < GC; ++i) gsum[i] = 0.f;
#pragma unroll
            for (int j = 0; j < KTPG; ++j)
#pragma unroll
                for (int i = 0; i < GC; ++i) gsum[i] += run_elem<false>(rg.la[j], i) * kLog2e;
#pragma unroll
            for (int i = 0; i < GC; ++i) incl[i] = gsum[i];
#pragma unroll
            for (int sft = KCP; sft < 64; sft *= 2)
#pragma unroll
                for (int i = 0; i < GC; ++i) {
                    const float y = lane_read(incl[i], lane - sft);
                    if (lane >= sft) incl[i] += y;
                }
#pragma unroll
            for (int i = 0; i < GC; ++i) {
                gexc[i] = incl[i] - gsum[i];
                wsum[i] = KCP < 64 ? lane_read(incl[i], 64 - KCP + lane % KCP) : incl[i];
                if constexpr (NW == 1) gmid[i] = lane_read(incl[i], (KTG / 2 - 1) * KCP + lane % KCP);
            }
#pragma unroll
            for (int i = GC; i < CW; ++i) {
                gexc[i] = gexc[0];
                wsum[i] = wsum[0];
                gmid[i] = gmid[0];
            }
            // the previous chunk is done with every LDS tile (with two sets,
            // this chunk's set was last read before the previous barrier)
            if constexpr (NBUF == 1) __syncthreads();
            if (lane < KCP) lds_store_words<CW>(&sm.tot[bsel][wave][CW * kcp], pack_run<false, CW>(wsum));
            if constexpr (Cfg::VGM) {
                // for the sub-chunk path: the in-wave prefix at each block's
                // eighth and last token, left by the run that ends there
                float ginc[CW];
#pragma unroll
                for (int i = 0; i < CW; ++i) ginc[i] = i < GC ? incl[i] : incl[0];
                if constexpr (SUB) {
                    const int e = ((ktg + 1) * KTPG) % 16;
                    if (e == 8) lds_store_words<CW>(&sm.bmid[(ktg * KTPG) / 16][CW * kcp], pack_run<false, CW>(ginc));
                    if (e == 0) lds_store_words<CW>(&sm.bend[(ktg * KTPG) / 16][CW * kcp], pack_run<false, CW>(ginc));
                }
                // this wave's vote: a channel's sum over the wave's tokens
                // beyond what the chunk-middle factors allow
                bool bad = false;
#pragma unroll
                for (int i = 0; i < GC; ++i) bad = bad || wsum[i] < Cfg::WAVE_THR;
                const bool wbad = __builtin_amdgcn_ballot_w64(bad) != 0;
                if (lane == 0) sm.wslow[wave] = wbad ? 1 : 0;
            }
        }
        // NONE/GAMMA: the previous chunk is done with every LDS tile (not
        // needed with two sets).  DIAG: the wave sums are visible.
        if constexpr (VG || NBUF == 1) __syncthreads();

        // this group's offset (exclusive prefix over the chunk), the
        // chunk-middle reference and the chunk total, in log2 units
        float gref[CW], gtot[CW], goff[CW];
#pragma unroll
        for (int i = 0; i < CW; ++i) gref[i] = gtot[i] = goff[i] = 0.f;
        // sub-chunk path (a chunk whose gates are too strong for the
        // chunk-middle reference): each 16-token block j is factorised around
        // m_j, its cumulative log2-gate at its eighth token; e2 = e^{E_j - m_j}
        // with E_j the value at its last token.  The fast path has e2 = 1.
        int slow = 0;
        float e2[CW];
#pragma unroll
        for (int i = 0; i < CW; ++i) e2[i] = 1.f;
        if constexpr (VG) {
            // all wave sums are read before any is used, so the reads overlap
            float x[NW][CW];
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                const float* tv = &sm.tot[bsel][w2][CW * kcp];
                if constexpr (GATE == LA_GATE_SCALAR) {
#pragma unroll
                    for (int i = 0; i < CW; ++i) x[w2][i] = tv[0];
                } else if constexpr (CW == 4) {
                    const float4 v4 = *reinterpret_cast<const float4*>(tv);
                    x[w2][0] = v4.x; x[w2][1] = v4.y; x[w2][2] = v4.z; x[w2][3] = v4.w;
                } else {
                    const float2 v2 = *reinterpret_cast<const float2*>(tv);
                    x[w2][0] = v2.x; x[w2][1] = v2.y;
                }
            }
            float wpre[CW];
#pragma unroll
            for (int i = 0; i < CW; ++i) wpre[i] = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                if (w2 == wave_u) {   // uniform: the earlier waves' total
#pragma unroll
                    for (int i = 0; i < CW; ++i) wpre[i] = gtot[i];
                }
#pragma unroll
                for (int i = 0; i < CW; ++i) gtot[i] += x[w2][i];
                if (NW > 1 && w2 == NW / 2 - 1) {
#pragma unroll
                    for (int i = 0; i < CW; ++i) gref[i] = gtot[i];
                }
            }
#pragma unroll
            for (int i = 0; i < CW; ++i) {
                goff[i] = wpre[i] + gexc[i];
                if constexpr (NW == 1) gref[i] = gmid[i];
            }
            if constexpr (Cfg::VGM) {
                int f = 0;
#pragma unroll
                for (int w2 = 0; w2 < NW; ++w2) f |= sm.wslow[w2];
                f = __builtin_amdgcn_readfirstlane(f);
                if constexpr (SUB) slow = f;
                else if (f) return false;   // the sub-chunk kernel takes the segment
                if (SUB && slow) {
                    // references of this run's block j: m_j, E_j and the
                    // block's start B_j = E_{j-1} (0 for the first), each a
                    // fixed sum of wave totals plus an in-wave prefix
                    const int jown = (ktg * KTPG) / 16;
                    float m[CW], e[CW], b0[CW], run[CW];
#pragma unroll
                    for (int i = 0; i < CW; ++i) m[i] = e[i] = b0[i] = run[i] = 0.f;
                    // run = total of the waves before w2; a block's eighth
                    // and last token fall in known waves
#pragma unroll
                    for (int w2 = 0; w2 < NW; ++w2) {
#pragma unroll
                        for (int jb = 0; jb < TB; ++jb) {
                            if ((16 * jb + 7) / Cfg::TPW == w2 && jb == jown) {
                                const float* mv = &sm.bmid[jb][CW * kcp];
#pragma unroll
                                for (int i = 0; i < CW; ++i) m[i] = run[i] + mv[i];
                            }
                            if ((16 * jb + 15) / Cfg::TPW == w2 && (jb == jown || jb + 1 == jown)) {
                                const float* ev = &sm.bend[jb][CW * kcp];
#pragma unroll
                                for (int i = 0; i < CW; ++i) {
                                    const float ej = run[i] + ev[i];
                                    if (jb == jown) e[i] = ej;
                                    else b0[i] = ej;
                                }
                            }
                        }
#pragma unroll
                        for (int i = 0; i < CW; ++i) run[i] += x[w2][i];
                    }
#pragma unroll
                    for (int i = 0; i < CW; ++i) {
                        gref[i] = m[i];
                        e2[i] = __builtin_amdgcn_exp2f(e[i] - m[i]);
                    }
                    // the run at a block's start leaves the block's state
                    // factors: e^{m_j - B_j} before its state term and
                    // e^{E_j - m_j} after it (both at most one)
                    if ((ktg * KTPG) % 16 == 0) {
                        float fa[CW];
#pragma unroll
                        for (int i = 0; i < CW; ++i) fa[i] = __builtin_amdgcn_exp2f(m[i] - b0[i]);
                        lds_store_words<CW>(&sm.sa[jown][CW * kcp], pack_run<false, CW>(fa));
                        lds_store_words<CW>(&sm.sb[jown][CW * kcp], pack_run<false, CW>(e2));
                    }
                }
            }
        }
        const float egam = seg_g;   // gamma^(tokens after this chunk), backward walk
        if constexpr (GATE == LA_GATE_GAMMA) seg_g *= sm.gpow[clen];

        // ---- a1: features and decay factors, written to the LDS tiles, one
        // token at a time; the transposed runs are packed as they go
        {
            static_assert(KTPG % 2 == 0 && VTPG % 2 == 0, "transposed runs are whole token pairs");
            using W = typename Cfg::Pair;   // two consecutive tokens of one channel
            W kp[CW][KTPG / 2];
            float bcur[CW], prev[CW];
#pragma unroll
            for (int i = 0; i < CW; ++i) {
                bcur[i] = goff[i];
                prev[i] = 0.f;
            }
#pragma unroll
            for (int j = 0; j < KTPG; ++j) {
                const int t = ktg * KTPG + j;
                const bool ok = t < clen;
                float qv[CW], kv[CW];
                float ftok = 1.f;
                if constexpr (GATE == LA_GATE_GAMMA)
                    ftok = ok ? sm.gpow[REV ? t + 1 : clen - 1 - t] * (BACKAGG ? egam : 1.f) : 0.f;
                // scalar gate: the token's factors, once for all its channels
                float sq = 1.f, sk = 1.f, st = 1.f;
                if constexpr (GATE == LA_GATE_SCALAR) {
                    bcur[0] += run_elem<false>(rg.la[j], 0) * kLog2e;
                    const float d = bcur[0] - gref[0];
                    sq = __builtin_amdgcn_exp2f(d);
                    sk = __builtin_amdgcn_exp2f(-d);
                    st = REV ? sq : sk * e2[0];
                    if constexpr (BACKAGG) st = __builtin_amdgcn_exp2f(gtot[0] - bcur[0] + eacc[0]);
                }
#pragma unroll
                for (int i = 0; i < CW; ++i) {
                    float ka = run_elem<BF16>(rg.k[j], i);
                    if constexpr (ELU1) ka = elu1f(ka);
                    ka = ok ? ka : 0.f;
                    float fq = 1.f, fk = 1.f, ft = ftok;
                    if constexpr (GATE == LA_GATE_SCALAR) {
                        fq = sq;
                        fk = sk;
                        ft = st;
                    } else if constexpr (VG) {
                        bcur[i] += run_elem<false>(rg.la[j], i) * kLog2e;
                        const float d = bcur[i] - gref[i];
                        fq = __builtin_amdgcn_exp2f(d);
                        fk = __builtin_amdgcn_exp2f(-d);
                        ft = REV ? fq : fk * e2[i];
                        // backward walk: k e^{B - b} times the decay after the chunk
                        if constexpr (BACKAGG) ft = __builtin_amdgcn_exp2f(gtot[i] - bcur[i] + eacc[i]);
                    }
                    if constexpr (!SONLY) {
                        float qa = run_elem<BF16>(qreg[j], i);
                        if constexpr (ELU1) qa = elu1f(qa);
                        qv[i] = qa * fq;
                        kv[i] = ka * fk;
                    }
                    const float x = ka * ft;
                    if (j & 1) kp[i][j / 2] = T::pack(prev[i], x);
                    else prev[i] = x;
                }
                if constexpr (!SONLY) {
                    const int pos = qk_pos<Cfg>(t, CW * kcp);
                    lds_store_words(&sm.q[t][pos], pack_run<BF16, CW>(qv));
                    lds_store_words(&sm.k[t][pos], pack_run<BF16, CW>(kv));
                }
            }
#pragma unroll
            for (int i = 0; i < CW; ++i)
                store_pairs<Cfg, KTPG>(&sm.kt[bsel][CW * kcp + i][0], CW * kcp + i, ktg * KTPG, kp[i]);
            // V^T: regroup the loaded channel runs into token pairs
            W vp[VW][VTPG / 2];
#pragma unroll
            for (int m = 0; m < VTPG / 2; ++m)
#pragma unroll
                for (int i = 0; i < VW; ++i) vp[i][m] = token_pair<Cfg>(rg.v[2 * m], rg.v[2 * m + 1], i);
#pragma unroll
            for (int i = 0; i < VW; ++i)
                store_pairs<Cfg, VTPG>(&sm.vt[bsel][VW * vcp + i][0], VW * vcp + i, vtg * VTPG, vp[i]);
            if constexpr (BACKAGG && VG) {
#pragma unroll
                for (int i = 0; i < CW; ++i) eacc[i] += gtot[i];
            }
            if (ktg == 0) {
                // per-row state factors: DIAG applies post(previous) * pre(this)
                // before the chunk; GAMMA applies gamma^c after op2; the
                // backward walk leaves the accumulated state unscaled
                float sc[CW], pr[CW], po[CW];
#pragma unroll
                for (int i = 0; i < CW; ++i) sc[i] = pr[i] = po[i] = 1.f;
                if constexpr (VG) {
#pragma unroll
                    for (int i = 0; i < CW; ++i) {
                        const int row = CW * kcp + i;
                        sm.segsum[row] += gtot[i];
                        // the sub-chunk path keeps the true state between its
                        // blocks (it applies the previous chunk's after-factor
                        // only)
                        if constexpr (!BACKAGG) {
                            if (!(SUB && slow)) {
                                pr[i] = __builtin_amdgcn_exp2f(REV ? gtot[i] - gref[i] : gref[i]);
                                po[i] = __builtin_amdgcn_exp2f(REV ? gref[i] : gtot[i] - gref[i]);
                            }
                        }
                        sc[i] = sm.post[NBUF > 1 ? bsel ^ 1 : 0][row] * pr[i];
                    }
                } else if constexpr (GATE == LA_GATE_GAMMA && !BACKAGG) {
#pragma unroll
                    for (int i = 0; i < CW; ++i) sc[i] = pr[i] = sm.gpow[clen];
                }
                lds_store_words<CW>(&sm.scale[bsel][CW * kcp], pack_run<false, CW>(sc));
                lds_store_words<CW>(&sm.pre[bsel][CW * kcp], pack_run<false, CW>(pr));
                lds_store_words<CW>(&sm.post[bsel][CW * kcp], pack_run<false, CW>(po));
            }
        }

        // ---- refill the registers: q with chunk c + 1, this set with c + PD.
        // The waves with fewer op1 tiles issue theirs after their tiles,
        // where they would otherwise wait for the others
        constexpr int NTILE = TB * (TB + 1) / 2;
        const bool late = !SONLY && NTILE % NW != 0 && wave_u >= NTILE % NW;
        auto refill = [&]() {
            if constexpr (!Cfg::PREFETCH) return;
            if (ci + 1 < c_end) load_q(cof(ci + 1));
            if (ci + Cfg::PD < c_end) load_chunk(cof(ci + Cfg::PD), rg);
        };
        if (!late) refill();
        __syncthreads();

        // ---- op1: P^T = Kh Qh^T on the lower-triangular tiles; each lane
        // gets four consecutive s of one row t and writes them packed
        if constexpr (!SONLY) {
            auto score_tile = [&](int tb, int sb) {
                f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
                const int rs = 16 * sb + r, rt = 16 * tb + r;
#pragma unroll
                for (int kk = 0; kk < DK / MK; ++kk) {
                    const int pp = kk * MK + KPL * g;  // this lane's k-slots (permuted order)
                    const Frag a = T::load(&sm.k[rs][qk_phys<Cfg>(rs, pp)]);
                    const Frag b = T::load(&sm.q[rt][qk_phys<Cfg>(rt, pp)]);
                    acc = T::mma(a, b, acc);
                }
                float x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int s = 16 * sb + 4 * g + i;
                    float val = acc[i];
                    if (s > rt) val = 0.f;
                    else if constexpr (GATE == LA_GATE_GAMMA) val *= sm.gpow[rt - s];
                    x[i] = val;
                }
                store_run<BF16, 4>(&sm.p[rt][p_pos<Cfg>(rt, 16 * sb + 4 * g)], x);
                if constexpr (SUB) mfma_drain();
            };
            if (!(SUB && slow)) {
                int idx = 0;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
                    for (int sb = 0; sb <= tb; ++sb, ++idx) {
                        if (idx % NW != wave) continue;
                        score_tile(tb, sb);
                    }
                }
            } else {
                // sub-chunk path: the diagonal tiles only; a bf16 contraction
                // over s spans two blocks, so an odd block's row also reads
                // the tile to its left, which is cleared here
#pragma unroll
                for (int j = 0; j < TB; ++j) {
                    if (j % NW != wave) continue;
                    score_tile(j, j);
                    if (BF16 && (j & 1)) {
                        const float z4[4] = {0.f, 0.f, 0.f, 0.f};
                        const int rt = 16 * j + r;
                        store_run<BF16, 4>(&sm.p[rt][p_pos<Cfg>(rt, 16 * (j - 1) + 4 * g)], z4);
                    }
                }
            }
            if (late) refill();
            __syncthreads();

            // ---- a4: normaliser of each row, read with the state before this chunk
            if (norm && SUB && slow) {
                // sub-chunk path: z entering each block (times the block's
                // before-factor, as its state term reads the state), then
                // each row from its block's diagonal tile
                if (tid < DK) {
                    float zz = sm.z[tid];
#pragma unroll
                    for (int j = 0; j < TB; ++j) {
                        const float fa = sm.sa[j][tid], fb = sm.sb[j][tid];
                        sm.zs[j][tid] = fa * zz;
                        float cs = 0.f;
                        for (int s2 = 16 * j; s2 < 16 * j + 16; ++s2)
                            cs += T::tof(sm.kt[bsel][tid][tr_pos<Cfg>(tid, s2)]);
                        zz = fb * fa * zz + cs;
                    }
                    sm.z[tid] = zz;
                }
                __syncthreads();
                for (int t = tid; t < C; t += Cfg::NT) {
                    const int j = t / 16;
                    float rsum = 0.f;
                    for (int s2 = 16 * j; s2 <= t; ++s2) rsum += T::tof(sm.p[t][p_pos<Cfg>(t, s2)]);
                    float dq = 0.f;
                    for (int i = 0; i < DK; ++i) dq += T::tof(sm.q[t][qk_pos<Cfg>(t, i)]) * sm.zs[j][i];
                    sm.den[t] = dq + rsum;
                }
                __syncthreads();
            } else if (norm) {
                // row t: sum_{s<=t} P[t][s] + (decayed q_t) . z, split over
                // the NRL lanes of an aligned group (interleaved columns and
                // channels) and added up by DPP moves inside the group
                // (fixed trip counts, unrolled: reads in flight together)
                const int part = tid % NRL;
                for (int t = tid / NRL; t < C; t += Cfg::NT / NRL) {
                    float rsum = 0.f;
#pragma unroll NUNR
                    for (int n = 0; n < C / NRL; ++n) {
                        const int s = part + n * NRL;
                        const float x = T::tof(sm.p[t][p_pos<Cfg>(t, s)]);
                        rsum += s <= t ? x : 0.f;
                    }
                    float dq = 0.f;
#pragma unroll NUNR
                    for (int n = 0; n < DK / NRL; ++n) {
                        const int i = part + n * NRL;
                        float zz = sm.z[i];
                        if constexpr (VG) zz *= sm.pre[bsel][i];
                        dq += T::tof(sm.q[t][qk_pos<Cfg>(t, i)]) * zz;
                    }
                    if constexpr (GATE == LA_GATE_GAMMA) dq *= sm.gpow[t + 1];
                    const float den = lane_group_sum<NRL>(dq + rsum);
                    if (part == 0) sm.den[t] = den;
                }
                __syncthreads();
            }
        }
        // z <- post * (pre * z + sum_s Kt[:, s]): channel i over the NCL lanes
        // of an aligned group, added up by DPP moves
        if (norm && !(SUB && slow)) {
            const int i = tid / NCL, part = tid % NCL;
            if (i < DK) {
                float cs = 0.f;
#pragma unroll NUNR
                for (int n = 0; n < C / NCL; ++n) cs += T::tof(sm.kt[bsel][i][tr_pos<Cfg>(i, part + n * NCL)]);
                cs = lane_group_sum<NCL>(cs);
                if (part == 0) sm.z[i] = sm.post[bsel][i] * (sm.pre[bsel][i] * sm.z[i] + cs);
            }
        }

        // ---- value fragments: A operand of op2 and B operand of op3
        Frag vf[CP / MK][NB];
#pragma unroll
        for (int kk = 0; kk < CP / MK; ++kk)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = colbase + 16 * nb + r;
                vf[kk][nb] = T::load(&sm.vt[bsel][row][tr_pos<Cfg>(row, kk * MK + KPL * g)]);
            }

        if constexpr (VG) scale_rows<Cfg>(accS, sm.scale[bsel], g);

        if constexpr (!SONLY) {
            // ---- op2: O^T = S'^T Qh^T (+ per-token decay) + V^T P^T
            f32x4_t accO[NB][TB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) accO[nb][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if (!(SUB && slow)) {
                if constexpr (BF16) {
    #pragma unroll
                    for (int k2 = 0; k2 < DK / 32; ++k2) {
                        Frag as[NB];
    #pragma unroll
                        for (int nb = 0; nb < NB; ++nb) {
                            const float x[8] = {accS[2 * k2][nb][0], accS[2 * k2][nb][1],
                                                accS[2 * k2][nb][2], accS[2 * k2][nb][3],
                                                accS[2 * k2 + 1][nb][0], accS[2 * k2 + 1][nb][1],
                                                accS[2 * k2 + 1][nb][2], accS[2 * k2 + 1][nb][3]};
                            as[nb] = T::from8(x);
                        }
    #pragma unroll
                        for (int tb = 0; tb < TB; ++tb) {
                            const int t = 16 * tb + r;
                            // one unit of the permuted layout = state rows 4g.. and 16+4g..
                            const Frag b = T::load(&sm.q[t][qk_phys<Cfg>(t, 32 * k2 + 8 * g)]);
    #pragma unroll
                            for (int nb = 0; nb < NB; ++nb) accO[nb][tb] = T::mma(as[nb], b, accO[nb][tb]);
                        }
                    }
                } else {
    #pragma unroll
                    for (int mb = 0; mb < MB; ++mb)
    #pragma unroll
                        for (int i = 0; i < 4; ++i)
    #pragma unroll
                            for (int tb = 0; tb < TB; ++tb) {
                                const int t = 16 * tb + r;
                                const Frag b = sm.q[t][qk_pos<Cfg>(t, 16 * mb + 4 * g + i)];
    #pragma unroll
                                for (int nb = 0; nb < NB; ++nb)
                                    accO[nb][tb] = T::mma(accS[mb][nb][i], b, accO[nb][tb]);
                            }
                }
                if constexpr (GATE == LA_GATE_GAMMA) {
    #pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        const float f = sm.gpow[16 * tb + r + 1];
    #pragma unroll
                        for (int nb = 0; nb < NB; ++nb) accO[nb][tb] *= f;
                    }
                }
    #pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int t = 16 * tb + r;
    #pragma unroll
                    for (int kk = 0; kk <= (16 * tb + 15) / MK; ++kk) {
                        const Frag b = T::load(&sm.p[t][p_pos<Cfg>(t, kk * MK + KPL * g)]);
    #pragma unroll
                        for (int nb = 0; nb < NB; ++nb) accO[nb][tb] = T::mma(vf[kk][nb], b, accO[nb][tb]);
                    }
                }
            } else {
                // sub-chunk path: block by block, the true state S_j taken to
                // the block's reference (times e^{m_j - B_j}), its rows' state
                // term and in-block scores, stored, then S_{j+1} = e^{E_j - m_j}
                // (...) + Kt_j^T V_j over the block's own tokens.  A compact
                // loop: one block's accumulators live at a time and the value
                // operands are read again from LDS.
                auto vfrag = [&](int kk, int nb) {
                    const int row = colbase + 16 * nb + r;
                    return T::load(&sm.vt[bsel][row][tr_pos<Cfg>(row, kk * MK + KPL * g)]);
                };
#pragma unroll 1
                for (int j = 0; j < TB; ++j) {
                    const int t = 16 * j + r;
                    f32x4_t acc[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                    scale_rows<Cfg>(accS, sm.sa[j], g);
                    if constexpr (BF16) {
#pragma unroll
                        for (int k2 = 0; k2 < DK / 32; ++k2) {
                            const Frag b = T::load(&sm.q[t][qk_phys<Cfg>(t, 32 * k2 + 8 * g)]);
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb) {
                                const float x[8] = {accS[2 * k2][nb][0], accS[2 * k2][nb][1],
                                                    accS[2 * k2][nb][2], accS[2 * k2][nb][3],
                                                    accS[2 * k2 + 1][nb][0], accS[2 * k2 + 1][nb][1],
                                                    accS[2 * k2 + 1][nb][2], accS[2 * k2 + 1][nb][3]};
                                acc[nb] = T::mma(T::from8(x), b, acc[nb]);
                            }
                        }
                    } else {
#pragma unroll
                        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const Frag b = sm.q[t][qk_pos<Cfg>(t, 16 * mb + 4 * g + i)];
#pragma unroll
                                for (int nb = 0; nb < NB; ++nb) acc[nb] = T::mma(accS[mb][nb][i], b, acc[nb]);
                            }
                    }
                    // the k-blocks of the block's 16 tokens (one for bf16)
                    constexpr int KPB = 16 / MK > 0 ? 16 / MK : 1;
#pragma unroll
                    for (int u = 0; u < KPB; ++u) {
                        const int kk = (16 * j) / MK + u;
                        const Frag b = T::load(&sm.p[t][p_pos<Cfg>(t, kk * MK + KPL * g)]);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) acc[nb] = T::mma(vfrag(kk, nb), b, acc[nb]);
                    }
                    mfma_drain();
                    // the block's rows (group norm: statistics of these rows
                    // across the waves)
                    const float inv = __builtin_amdgcn_rcpf(sm.den[t]);
                    float gmean = 0.f, grstd = 1.f;
                    if constexpr (EPI) {
                        float s1 = 0.f, s2 = 0.f;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float o = acc[nb][i] * inv;
                                s1 += o;
                                s2 += o * o;
                            }
                        s1 += lane_read(s1, lane ^ 16);
                        s2 += lane_read(s2, lane ^ 16);
                        s1 += lane_read(s1, lane ^ 32);
                        s2 += lane_read(s2, lane ^ 32);
                        if (g == 0) sm.gnp[wave][t] = make_float2(s1, s2);
                        __syncthreads();
                        s1 = s2 = 0.f;
#pragma unroll
                        for (int w2 = 0; w2 < NW; ++w2) {
                            const float2 x = sm.gnp[w2][t];
                            s1 += x.x;
                            s2 += x.y;
                        }
                        gmean = s1 * (1.0f / DV);
                        grstd = __builtin_amdgcn_rsqf(fmaxf(s2 * (1.0f / DV) - gmean * gmean, 0.f) + p.gn_eps);
                        __syncthreads();   // every wave has read this block's sums
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const uint32_t off = ((uint32_t)(t0 + t) * DV + colbase + 16 * nb + 4 * g) * ES;
                        f32x4_t o = acc[nb] * inv;
                        if constexpr (EPI) {
                            const Words<OW> gw = buf_load_words<OW>(rgate, off);
                            const bool gated = p.gn_gate != nullptr;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float y = (o[i] - gmean) * grstd * gnw[nb][i] + gnb[nb][i];
                                const float ga = run_elem<BF16>(gw, i);
                                const float sw = ga * __builtin_amdgcn_rcpf(1.0f + __expf(-ga));
                                o[i] = gated ? y * sw : y;
                            }
                        }
                        if constexpr (BF16) {
                            const u32x2_t w = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
                            __builtin_amdgcn_raw_buffer_store_b64(w, roc, off, 0, 0);
                        } else {
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), roc, off, 0, 0);
                        }
                    }
                    scale_rows<Cfg>(accS, sm.sb[j], g);
#pragma unroll
                    for (int mb = 0; mb < MB; ++mb) {
                        const int row = 16 * mb + r;
#pragma unroll
                        for (int u = 0; u < KPB; ++u) {
                            const int kk = (16 * j) / MK + u;
                            Frag a = T::load(&sm.kt[bsel][row][tr_pos<Cfg>(row, kk * MK + KPL * g)]);
                            // a bf16 contraction spans blocks 2kk and 2kk+1
                            // (lane groups 0-1 and 2-3): keep block j's half
                            if constexpr (MK > 16) {
                                if ((g >> 1) != (j & 1)) a = __builtin_bit_cast(Frag, make_uint4(0u, 0u, 0u, 0u));
                            }
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb) accS[mb][nb] = T::mma(a, vfrag(kk, nb), accS[mb][nb]);
                        }
                    }
                    mfma_drain();
                }
            }
            // ---- store: lane (r, g) holds 4 consecutive columns of token row t
            // (the sub-chunk path has stored its rows block by block)
            float gmean[EPI ? TB : 1], grstd[EPI ? TB : 1];
            if (!(SUB && slow)) {
            if constexpr (EPI) {
                // group norm statistics of each token's d_v outputs: the
                // lane's 4 NB values, the 4 lanes of the token in this wave,
                // then the waves through LDS
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const float inv = __builtin_amdgcn_rcpf(sm.den[16 * tb + r]);
                    float s1 = 0.f, s2 = 0.f;
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float o = accO[nb][tb][i] * inv;
                            s1 += o;
                            s2 += o * o;
                        }
                    s1 += lane_read(s1, lane ^ 16);
                    s2 += lane_read(s2, lane ^ 16);
                    s1 += lane_read(s1, lane ^ 32);
                    s2 += lane_read(s2, lane ^ 32);
                    if (g == 0) sm.gnp[wave][16 * tb + r] = make_float2(s1, s2);
                }
                __syncthreads();
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    float s1 = 0.f, s2 = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < NW; ++w2) {
                        const float2 x = sm.gnp[w2][16 * tb + r];
                        s1 += x.x;
                        s2 += x.y;
                    }
                    const float mean = s1 * (1.0f / DV);
                    const float var = fmaxf(s2 * (1.0f / DV) - mean * mean, 0.f);
                    gmean[tb] = mean;
                    grstd[tb] = __builtin_amdgcn_rsqf(var + p.gn_eps);
                }
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const int t = 16 * tb + r;
                const float inv = __builtin_amdgcn_rcpf(sm.den[t]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const uint32_t off = ((uint32_t)(t0 + t) * DV + colbase + 16 * nb + 4 * g) * ES;
                    f32x4_t o = accO[nb][tb] * inv;
                    if constexpr (EPI) {
                        const bool gated = p.gn_gate != nullptr;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float y = (o[i] - gmean[tb]) * grstd[tb] * gnw[nb][i] + gnb[nb][i];
                            const float a = run_elem<BF16>(greg[nb][tb], i);
                            const float sw = a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
                            o[i] = gated ? y * sw : y;
                        }
                    }
                    if constexpr (BF16) {
                        const u32x2_t w = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
                        __builtin_amdgcn_raw_buffer_store_b64(w, roc, off, 0, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, o), roc, off, 0, 0);
                    }
                }
            }
            }
        }

        if constexpr (EPI) {
            if (ci + 1 < c_end) load_gate(cof(ci + 1));
        }

        // ---- op3: state update (the sub-chunk path has done it block by block)
        if constexpr (GATE == LA_GATE_GAMMA) scale_rows<Cfg>(accS, sm.scale[bsel], g);
        if (!(SUB && slow)) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int row = 16 * mb + r;
#pragma unroll
                for (int kk = 0; kk < CP / MK; ++kk) {
                    const Frag a = T::load(&sm.kt[bsel][row][tr_pos<Cfg>(row, kk * MK + KPL * g)]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) accS[mb][nb] = T::mma(a, vf[kk][nb], accS[mb][nb]);
                }
            }
        }
        // ---- the state at the next chunk boundary (the entry state of the
        // next segment is stored by that segment's workgroup)
        if constexpr (STORE) {
            const int nxt = c + 1;
            if (nxt < c_end || seg == P - 1) store_state(nxt, bsel);
        }
        // the loop's back-edge follows: the compiler's wait states after the
        // last state products do not always survive it (the assembly check
        // finds it in the sub-chunk kernels and, with d < 128, in the
        // vector-gate main passes)
        if constexpr (SUB || (Cfg::VGM && DK < 128)) mfma_drain();
        return true;
    };
    if constexpr (STORE) {
        // the segment's entry state is the first boundary it owns (the
        // diagonal after-factor of a previous chunk is 1 here)
        if (c_begin < c_end) {
            __syncthreads();   // sm.post set up
            store_state(c_begin, 0);
        }
    }
    {
        if (Cfg::PREFETCH && c_begin < c_end) load_q(cof(c_begin));
        if (c_begin < c_end) load_gate(cof(c_begin));
        if constexpr (Cfg::PD == 2) {
            ChunkRegs ra, rb;
            if (c_begin < c_end) load_chunk(cof(c_begin), ra);
            if (c_begin + 1 < c_end) load_chunk(cof(c_begin + 1), rb);
            for (int ci = c_begin; ci < c_end; ci += 2) {
                step(ci, ra);
                if (ci + 1 < c_end) step(ci + 1, rb);
            }
        } else {
            ChunkRegs ra;
            if (Cfg::PREFETCH && c_begin < c_end) load_chunk(cof(c_begin), ra);
            bool done = true;
            for (int ci = c_begin; ci < c_end; ++ci)
                if (!step(ci, ra)) {
                    done = false;
                    break;
                }
            if constexpr (Cfg::VGM && !ROB) {
                // every segment records whether it was handed over
                if (tid == 0) *seg_flag = done ? 0 : 1;
                if (!done) return;
            }
        }
    }
    // DIAG: the last chunk's after-factor (in the set of the last chunk
    // walked; both sets hold ones before the first)
    if constexpr (VG) {
        __syncthreads();
        scale_rows<Cfg>(accS, sm.post[NBUF > 1 ? (c_end - 1) & 1 : 0], g);
    }

    // ---- epilogue
    float* Sout;
    float* zout;
    if constexpr (STORE && SONLY) {
        // the state after the whole sequence, from its last segment
        if (seg != P - 1) return;
        Sout = p.S_final ? p.S_final + (size_t)bh * SS : nullptr;
        zout = nullptr;
    } else if constexpr (SONLY) {
        Sout = p.ws_S + ((size_t)bh * P + seg) * SS;
        zout = p.ws_z + ((size_t)bh * P + seg) * DK;
        float* aout = p.ws_a + ((size_t)bh * P + seg) * DK;
        if constexpr (VG) {
            if (tid < DK) aout[tid] = __builtin_amdgcn_exp2f(sm.segsum[tid]);
        } else {
            if (tid < DK) aout[tid] = GATE == LA_GATE_GAMMA ? seg_g : 1.0f;
        }
    } else {
        if (seg != P - 1) return;
        Sout = p.S_final ? p.S_final + (size_t)bh * SS : nullptr;
        zout = p.z_final ? p.z_final + (size_t)bh * DK : nullptr;
    }
    if (Sout) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sout[(size_t)(16 * mb + 4 * g + i) * DV + colbase + 16 * nb + r] = accS[mb][nb][i];
    }
    if (norm && zout && tid < DK) zout[tid] = sm.z[tid];
}

// Segment scan: S_in[0] = S0, S_in[j+1] = a_j * S_in[j] + U_j, written in
// place over the workspace slots (slot j holds U_j on entry, S_in[j] on exit).
// Only the multiply-adds are sequential: each thread reads a batch of its
// segment slots and factors before running the chain over them, so the
// memory latency is paid once per batch rather than once per segment.
// With REV the scan runs from the last segment to the first: slot P-1
// starts from the initial value (S0 holds it) and G_in[j] = a_{j+1} *
// G_in[j+1] + U_{j+1}, the composition of the gradient recurrence.
template <int DK, int DV, bool REV = false>
__global__ __launch_bounds__(256) void state_scan_kernel(const ChunkParams p) {
    constexpr int N4 = DK * DV / 4;
    constexpr int NBX = (N4 + 255) / 256;
    constexpr int NBATCH = 8;
    const int bh = blockIdx.x / NBX;
    const int bx = blockIdx.x % NBX;
    const int e4 = bx * 256 + threadIdx.x;
    const int P = p.P;
    const size_t SS = (size_t)DK * DV;
    if (e4 < N4) {
        const int row = (e4 * 4) / DV;
        float4 x = p.S0 ? reinterpret_cast<const float4*>(p.S0 + (size_t)bh * SS)[e4]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        float4* slots = reinterpret_cast<float4*>(p.ws_S + (size_t)bh * P * SS) + e4;
        const float* as = p.ws_a + (size_t)bh * P * DK + row;
        // position k of the chain reads and writes slot sj(k)
        auto sj = [&](int k) { return REV ? P - 1 - k : k; };
        for (int j0 = 0; j0 < P - 1; j0 += NBATCH) {
            float4 u[NBATCH];
            float a[NBATCH];
#pragma unroll
            for (int jj = 0; jj < NBATCH; ++jj) {
                if (j0 + jj < P - 1) {
                    u[jj] = slots[(size_t)sj(j0 + jj) * (SS / 4)];
                    a[jj] = as[(size_t)sj(j0 + jj) * DK];
                }
            }
#pragma unroll
            for (int jj = 0; jj < NBATCH; ++jj) {
                if (j0 + jj < P - 1) {
                    slots[(size_t)sj(j0 + jj) * (SS / 4)] = x;
                    x = make_float4(a[jj] * x.x + u[jj].x, a[jj] * x.y + u[jj].y,
                                    a[jj] * x.z + u[jj].z, a[jj] * x.w + u[jj].w);
                }
            }
        }
        slots[(size_t)sj(P - 1) * (SS / 4)] = x;
    }
    if (p.normalize && bx == 0 && threadIdx.x < DK) {
        const int i = threadIdx.x;
        float zx = p.z0 ? p.z0[(size_t)bh * DK + i] : 0.f;
        float* zs = p.ws_z + (size_t)bh * P * DK + i;
        const float* as = p.ws_a + (size_t)bh * P * DK + i;
        for (int j0 = 0; j0 < P - 1; j0 += NBATCH) {
            float u[NBATCH], a[NBATCH];
#pragma unroll
            for (int jj = 0; jj < NBATCH; ++jj) {
                if (j0 + jj < P - 1) {
                    u[jj] = zs[(size_t)(j0 + jj) * DK];
                    a[jj] = as[(size_t)(j0 + jj) * DK];
                }
            }
#pragma unroll
            for (int jj = 0; jj < NBATCH; ++jj) {
                if (j0 + jj < P - 1) {
                    zs[(size_t)(j0 + jj) * DK] = zx;
                    zx = a[jj] * zx + u[jj];
                }
            }
        }
        zs[(size_t)(P - 1) * DK] = zx;
    }
}

// Waves per workgroup for a state width: 32 state columns per wave at 128,
// 16 otherwise.
template <int D>
struct ChunkWaves {
    static constexpr int value = D >= 128 ? 8 : (D / 16 < 4 ? D / 16 : 4);
};

// Host-side dispatch over chunk length, gate mode and pass for one (d, dtype).
// The backward passes exist for the backward's chunk length only.
// dk != dv (64 and 128 either way, bf16): the waves of the narrower width,
// and neither the backward's passes nor the 128-token tile.
template <int DK, int DV, bool BF, int NWV = ChunkWaves<(DK < DV ? DK : DV)>::value>
hipError_t launch_chunk_dt(const ChunkParams& p, int chunk, int gate, int pass, hipStream_t s,
                           int nblocks, bool robust) {
    constexpr int D = DK;
    constexpr bool SQUARE = DK == DV;
#define LA_CHUNK_LAUNCH(CC, GG, SO, RV, ST, EP, RB)                                        \
    do {                                                                                   \
        using Cfg = ChunkCfg<DK, DV, CC, BF, GG, SO, NWV>;                                 \
        if (p.phi_elu1)                                                                    \
            LA_LAUNCH((chunk_kernel<Cfg, true, RV, ST, EP, RB>), dim3(nblocks), dim3(Cfg::NT), s, p); \
        else                                                                               \
            LA_LAUNCH((chunk_kernel<Cfg, false, RV, ST, EP, RB>), dim3(nblocks), dim3(Cfg::NT), s, p); \
        return hipGetLastError();                                                          \
    } while (0)
// main passes under a vector gate exist twice: without and with the
// sub-chunk path (robust)
#define LA_CHUNK_GATES_EP(CC, SO, RV, ST, EP)                                           \
    do {                                                                                \
        if (gate == LA_GATE_NONE) LA_CHUNK_LAUNCH(CC, 0, SO, RV, ST, EP, false);        \
        if (gate == LA_GATE_GAMMA) LA_CHUNK_LAUNCH(CC, 1, SO, RV, ST, EP, false);       \
        if constexpr (SO) {                                                             \
            if (gate == LA_GATE_DIAG) LA_CHUNK_LAUNCH(CC, 2, SO, RV, ST, EP, false);    \
            if (gate == LA_GATE_SCALAR) LA_CHUNK_LAUNCH(CC, 3, SO, RV, ST, EP, false);  \
        } else {                                                                        \
            if (gate == LA_GATE_DIAG && !robust) LA_CHUNK_LAUNCH(CC, 2, SO, RV, ST, EP, false); \
            if (gate == LA_GATE_DIAG && robust) LA_CHUNK_LAUNCH(CC, 2, SO, RV, ST, EP, true);   \
            if (gate == LA_GATE_SCALAR && !robust) LA_CHUNK_LAUNCH(CC, 3, SO, RV, ST, EP, false); \
            if (gate == LA_GATE_SCALAR && robust) LA_CHUNK_LAUNCH(CC, 3, SO, RV, ST, EP, true);   \
        }                                                                               \
    } while (0)
#define LA_CHUNK_GATES(CC, SO, RV, ST) LA_CHUNK_GATES_EP(CC, SO, RV, ST, false)
#define LA_CHUNK_FWD(CC)                                                 \
    do {                                                                 \
        if (pass == PASS_STATE) LA_CHUNK_GATES(CC, true, false, false);  \
        if (pass == PASS_MAIN) LA_CHUNK_GATES(CC, false, false, false);  \
    } while (0)
    // chunk lengths below a tile run in it (48 in the 64 tile; 80, 96 and
    // 112 in the 128 tile, which fits the LDS for bf16 at d <= 64 and fp32 at
    // d <= 32)
    const int tile = chunk <= 16 ? 16 : chunk <= 32 ? 32 : chunk <= 64 ? 64 : 128;
    constexpr int CB = bwd_chunk(D, BF);
    if constexpr (SQUARE) {
        if (chunk == CB) {
            if (pass == PASS_STATE_REV) LA_CHUNK_GATES(CB, true, true, false);
            if (pass == PASS_STORE) LA_CHUNK_GATES(CB, true, false, true);
            if (pass == PASS_MAIN_STORE) LA_CHUNK_GATES(CB, false, false, true);
        }
    }
    if (pass == PASS_MAIN_NORM && chunk == 64) LA_CHUNK_GATES_EP(64, false, false, false, true);
    if (tile == 16) LA_CHUNK_FWD(16);
    if (tile == 32) LA_CHUNK_FWD(32);
    if (tile == 64) LA_CHUNK_FWD(64);
    if constexpr (SQUARE && chunk_tile128<D, BF>()) {
        if (tile == 128) LA_CHUNK_FWD(128);
    }
    return hipErrorInvalidValue;
#undef LA_CHUNK_FWD
#undef LA_CHUNK_GATES
#undef LA_CHUNK_GATES_EP
#undef LA_CHUNK_LAUNCH
}

// One explicit (d, dtype) instantiation per translation unit.
#define LA_DEFINE_CHUNK_LAUNCHER(NAME, D, BF)                                                      \
    hipError_t NAME(const ChunkParams& p, int chunk, int gate, int pass, hipStream_t s,            \
                    int nblocks, bool robust) {                                                    \
        return launch_chunk_dt<D, D, BF>(p, chunk, gate, pass, s, nblocks, robust);                \
    }
// (d_k, d_v, dtype) with d_k != d_v.
#define LA_DEFINE_CHUNK_LAUNCHER_KV(NAME, DK, DV, BF)                                              \
    hipError_t NAME(const ChunkParams& p, int chunk, int gate, int pass, hipStream_t s,            \
                    int nblocks, bool robust) {                                                    \
        return launch_chunk_dt<DK, DV, BF>(p, chunk, gate, pass, s, nblocks, robust);              \
    }

}  // namespace la
