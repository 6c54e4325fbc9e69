// bwd_kernel.h -- gradients of the unified recurrence on gfx950 matrix
// cores: one workgroup walks a (b,h) segment of chunks from its last chunk
// to its first, carrying the gradient of the state through the walk.
//
// With S = the state before a chunk, G = the gradient of the state after
// it, chunk-local t, s, b_t = sum_{r<=t} log a_r (per key channel, natural
// log) and B = b at the chunk's last token, the forward chunk ("Module 22:
// Linear & Recurrent Attention", "The Three Faces of Retention", with the
// diagonal gate of "The One Recurrence Behind Them All") is
//   o_t = (q_t * e^{b_t})^T S + sum_{s<=t} [sum_i q_ti k_si e^{b_ti - b_si}] v_s
// and its reverse-mode derivative, written per chunk, is
//   dq_t = e^{b_t} * (S do_t) + sum_{s<=t} (do_t . v_s) k_s * e^{b_t - b_s}
//   dk_s = e^{B - b_s} * (G v_s) + sum_{t>=s} (do_t . v_s) q_t * e^{b_t - b_s}
//   dv_s = G^T (k_s * e^{B - b_s}) + sum_{t>=s} P[t][s] do_t
//   d log a_t = sum_{u>=t} (q_u * dq_u - k_u * dk_u)      (features q, k)
//   G_prev = e^{B} * G + sum_t (q_t * e^{b_t}) do_t^T     (the chunk before)
// where P[t][s] is the forward score with its decay.  The suffix sum that
// reaches into later chunks, sum over all tokens after this chunk, equals
// rowsum(G * S_next) with S_next the state after this chunk, so each chunk
// finishes its own d log a without a pass over the sequence.  S_next is not
// read: with S_next = e^{B} S + sum_s (k_s e^{B - b_s}) v_s^T,
//   rowsum(G * S_next)_i = e^{B_i} rowsum(G * S)_i
//                          + sum_s k_si e^{B_i - b_si} (G v_s)_i
// and G v_s is the first term of dk_s, already in the accumulators.
//
// Matrix-core mapping (C tokens, D = d_k = d_v; wave w owns channel block
// [16w, 16w+16) of dq, dk and of dv, and a block of G's tiles):
//   P   = Qh Kh^T and dP = dO V^T on the lower-triangular 16x16 tiles
//         (Qh = q e^{b - r}, Kh = k e^{r - b}, r = b at the chunk middle),
//         stored transposed, [s][t], with the causal mask (and gamma^(t-s));
//   dQ^T = e^{r} S dO^T + Kh^T dP^T,   then * e^{b - r}
//   dK^T = Gs V^T + Qh^T dP,           then * e^{r - b}
//   dV^T = Gs^T Kh^T + dO^T P
//   G_prev = e^{r} (Gs + Qh^T dO), formed as its transpose dO^T Qh
// with Gs = diag(e^{B - r}) G.  G stays in LDS in fp32 for the whole walk
// (row-major, 16-byte units swizzled by the row); where it is an operand
// it is read there, scaled by the row factor e^{B - r} and rounded to the
// element type.  S comes from memory in the element type.  q, k, v and dO
// are loaded in whole rows into their LDS tiles; each thread then takes
// one 4-channel run of q and k per owned token from there.  Every output
// lane of the gradient products holds 4 consecutive channels of one token,
// the same elements whose features and decay factors that thread formed;
// every output lane of the G step holds 4 consecutive columns of one row of
// G.  Operands with the token index (or G's row index) as the contraction
// are read from row-major LDS tiles with the transposing LDS read of gfx950
// (ds_read_b64_tr_b16).
#pragma once

#include "la_device.h"
#include "la_internal.h"
#include "tile_ops.h"

namespace la {

template <int D_, int C_, bool BF16_, int GATE_>
struct BwdCfg {
    static constexpr int D = D_, C = C_, GATE = GATE_;
    static constexpr bool BF16 = BF16_;
    using T = Elem<BF16>;
    using E = typename T::E;
    using Frag = typename T::Frag;
    static constexpr int NW = D / 16;                  // waves: one channel block each
    static constexpr int NT = 64 * NW;
    static constexpr int TB = C / 16;                  // token blocks
    static constexpr int KPL = T::KPL, MK = T::MK;
    static constexpr int UE = 16 / (int)sizeof(E);     // elements per 16-byte unit
    static constexpr int DU = D / UE, TU = C / UE;     // units per row
    // the D-wide tiles swizzle over up to 16 units (256 bytes): the LDS has
    // 64 four-byte banks, so 16 consecutive rows of a fragment read fall on
    // 16 different bank groups
    static constexpr int DMASK = (DU < 16 ? DU : 16) - 1;
    static constexpr int TMASK = (TU < 8 ? TU : 8) - 1;
    static constexpr int RW = 4 * (int)sizeof(E) / 4;  // words of a 4-channel run
    static_assert(D % 16 == 0 && C % MK == 0 && C % 16 == 0, "tile shape");
    static_assert(!BF16 || D % 32 == 0, "bf16 needs d >= 32");
};

template <class Cfg>
struct BwdSmem {
    using E = typename Cfg::E;
    alignas(16) E qh[Cfg::C][Cfg::D];     // Qh   [t][swizzled i]
    alignas(16) E kh[Cfg::C][Cfg::D];     // Kh   [s][swizzled i]
    alignas(16) E dout[Cfg::C][Cfg::D];   // dO   [t][swizzled n]
    alignas(16) E vv[Cfg::C][Cfg::D];     // V    [s][swizzled n]
    alignas(16) E pt[Cfg::C][Cfg::C];     // P^T  [s][swizzled t]
    alignas(16) E dpt[Cfg::C][Cfg::C];    // dP^T [s][swizzled t]
    alignas(16) float gm[Cfg::D * Cfg::D];  // G, fp32 [i][swizzled n]
    float red[Cfg::NW][Cfg::C];           // per-wave token sums (scalar gate)
    alignas(16) float ebr[Cfg::D];        // e^{B - r} per channel (DIAG)
    alignas(16) float er[Cfg::D];         // e^{r} per channel (DIAG)
    float gpow[Cfg::C + 2];               // gamma^j
};

// Operand from a state in memory (element type): rows r0..r0+15 (lane & 15),
// k-slots the row's elements k0 + (slots of this lane).
template <class Cfg>
__device__ __forceinline__ typename Cfg::Frag mem_frag(const typename Cfg::E* M, int ld, int r0,
                                                       int k0, int lane) {
    const int row = r0 + (lane & 15);
    const int col = k0 + Cfg::KPL * (lane >> 4);
    return Cfg::T::load(M + (size_t)row * ld + col);
}
// Position of (row, col) in the fp32 G tile: row-major, 16-byte units
// XOR-swizzled by the row.  For the bf16 kernel at d = 128 (512-byte rows)
// the unit XOR is (row & 3) | (r2 ^ r3) << 2 | r2 << 3 (r_i: bit i of the
// row): on gfx950 the column reads of G (4-byte reads of rows 8 apart, two
// passes of 32 lanes over 128 bytes of banks) were two-way bank-conflicted
// under row ^ row / 16, and this keeps the 16-row float4 reads and writes
// conflict-free as well.  Elsewhere row ^ row / 16, so that 16 consecutive
// rows, and rows 16 apart, fall on different banks.
template <class Cfg>
__device__ __forceinline__ int g_pos(int row, int col) {
    constexpr int D = Cfg::D;
    constexpr int U = D / 4;
    constexpr int M = (U < 16 ? U : 16) - 1;
    int x;
    if constexpr (Cfg::BF16 && D == 128)
        x = (row & 3) | ((((row >> 2) ^ (row >> 3)) & 1) << 2) | (((row >> 2) & 1) << 3);
    else
        x = (row ^ (row >> 4)) & M;
    return row * D + ((((col >> 2) ^ x) << 2) | (col & 3));
}

// The KPL k-slots of G's row `row` from column `col` on, as floats.
template <class Cfg>
__device__ __forceinline__ void g_row(const float* gm, int row, int col, float* x) {
    constexpr int D = Cfg::D;
    if constexpr (Cfg::BF16) {
        const float4 a = *reinterpret_cast<const float4*>(gm + g_pos<Cfg>(row, col));
        const float4 b = *reinterpret_cast<const float4*>(gm + g_pos<Cfg>(row, col + 4));
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
        x[0] = gm[g_pos<Cfg>(row, col)];
    }
}

// KPL floats -> one operand in the element type.
template <class Cfg>
__device__ __forceinline__ typename Cfg::Frag to_frag(const float* x) {
    if constexpr (Cfg::BF16) return Cfg::T::from8(x);
    else return x[0];
}

template <class Cfg, bool ELU1>
__global__ __launch_bounds__(Cfg::NT) void bwd_kernel(const BwdParams p) {
    constexpr int D = Cfg::D, C = Cfg::C, GATE = Cfg::GATE, TB = Cfg::TB, NW = Cfg::NW;
    constexpr int MK = Cfg::MK, RW = Cfg::RW, KPL = Cfg::KPL, UE = Cfg::UE, DU = Cfg::DU;
    constexpr bool BF16 = Cfg::BF16;
    constexpr int ES = (int)sizeof(typename Cfg::E);
    constexpr int DM = Cfg::DMASK, TM = Cfg::TMASK;
    using T = typename Cfg::T;
    using E = typename Cfg::E;
    using Frag = typename Cfg::Frag;
    constexpr float kLog2e = 1.4426950408889634f;
    // the diagonal and the per-token scalar gate share one path
    constexpr bool VG = GATE == LA_GATE_DIAG || GATE == LA_GATE_SCALAR;
    // float4 units of G each thread copies in (and out, for dS0)
    constexpr int GQ = D * D / 4 / Cfg::NT;
    // 16-byte units of a C x D tile each thread loads
    constexpr int VU = C * D / UE / Cfg::NT;
    static_assert(VU * UE * Cfg::NT == C * D, "tile load mapping");
    static_assert(GQ * 4 * Cfg::NT == D * D, "G copy mapping");

    __shared__ BwdSmem<Cfg> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int seg = blockIdx.x % p.P;
    const int bh = blockIdx.x / p.P;
    const int h = bh % p.H;
    const int L = p.L;
    const int c_begin = seg * p.cps;
    const int c_end = min(p.nchunks, c_begin + p.cps);
    const int nb = wave;                  // channel block of this wave

    const size_t rows0 = (size_t)bh * L;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const E*>(p.q) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const E*>(p.k) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const E*>(p.v) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rdo = make_rsrc(reinterpret_cast<const E*>(p.dout) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rla =
        make_rsrc(GATE == LA_GATE_DIAG ? (const void*)(p.log_alpha + rows0 * D)
                  : GATE == LA_GATE_SCALAR ? (const void*)(p.log_alpha + rows0) : p.q,
                  GATE == LA_GATE_DIAG ? (uint32_t)L * D * 4
                  : GATE == LA_GATE_SCALAR ? (uint32_t)L * 4 : 0u);
    const __amdgpu_buffer_rsrc_t rdq = make_rsrc(reinterpret_cast<E*>(p.dq) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rdk = make_rsrc(reinterpret_cast<E*>(p.dk) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rdv = make_rsrc(reinterpret_cast<E*>(p.dv) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rdla =
        make_rsrc(GATE == LA_GATE_DIAG ? (void*)(p.dlog_alpha + rows0 * D)
                  : GATE == LA_GATE_SCALAR ? (void*)(p.dlog_alpha + rows0) : p.dq,
                  GATE == LA_GATE_DIAG ? (uint32_t)L * D * 4
                  : GATE == LA_GATE_SCALAR ? (uint32_t)L * 4 : 0u);
    const E* Sbh = reinterpret_cast<const E*>(p.st_fwd) + (size_t)bh * (p.nchunks + 1) * D * D;

    if constexpr (GATE == LA_GATE_GAMMA) {
        const float l2g = p.log2_gamma[h];
        for (int j = tid; j < C + 2; j += Cfg::NT) sm.gpow[j] = j == 0 ? 1.0f : exp2f((float)j * l2g);
    }
    // zero the score tiles: only their lower-triangular 16x16 tiles are
    // ever written, and the rest is read as zeros
    {
        E* z0 = &sm.pt[0][0];
        E* z1 = &sm.dpt[0][0];
        for (int i = tid; i < C * C; i += Cfg::NT) {
            z0[i] = E(0);
            z1[i] = E(0);
        }
    }
    // G after the segment's last chunk (zeros without one); visible after
    // the first chunk's tile barrier
    {
        // all of this thread's loads in flight before the first LDS write
        float4 x[GQ];
        if (p.g_entry) {
            const float4* gin = reinterpret_cast<const float4*>(p.g_entry + ((size_t)bh * p.P + seg) * D * D);
#pragma unroll
            for (int j = 0; j < GQ; ++j) x[j] = gin[tid + j * Cfg::NT];
        } else {
#pragma unroll
            for (int j = 0; j < GQ; ++j) x[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            const int u = tid + j * Cfg::NT;
            *reinterpret_cast<float4*>(&sm.gm[g_pos<Cfg>(u / (D / 4), 4 * (u % (D / 4)))]) = x[j];
        }
    }

    for (int c = c_end - 1; c >= c_begin; --c) {
        // the lane index, opaque to the compiler in each chunk: otherwise the
        // many lane-dependent LDS and memory addresses of a chunk are hoisted
        // out of the walk and held in registers across it
        int lane = tid & 63;
        asm volatile("" : "+v"(lane));
        lane &= 63;
        const int r = lane & 15, g = lane >> 4;
        const int ch0 = 16 * wave + 4 * g;    // this thread's 4 channels (keys and values)
        const int t0 = c * C;
        const int clen = min(C, L - t0);
        const E* Sc = Sbh + (size_t)c * D * D;

        // ---- loads.  q, k, v and dO land in their LDS tiles first: whole
        // rows, 16 bytes a lane (a wave reading 16 tokens x 4 channels per
        // instruction would touch 16 rows for 32 bytes each, and the memory
        // pipeline's issue rate, not HBM, set the pace).  The gates come
        // as one 4-channel run per owned token.
        Words<4> lar[VG ? TB : 1];
        Words<4> qc[VU], kc[VU], vc[VU], dc[VU];
#pragma unroll
        for (int j = 0; j < VU; ++j) {
            const int u = tid + j * Cfg::NT;
            const uint32_t off = (uint32_t)t0 * D * ES + (uint32_t)u * 16;
            qc[j] = buf_load_words<4>(rq, off);
            kc[j] = buf_load_words<4>(rk, off);
            vc[j] = buf_load_words<4>(rv, off);
            dc[j] = buf_load_words<4>(rdo, off);
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const uint32_t row = (uint32_t)(t0 + 16 * tb + r);
            if constexpr (GATE == LA_GATE_DIAG) lar[tb] = buf_load_words<4>(rla, (row * D + ch0) * 4);
            if constexpr (GATE == LA_GATE_SCALAR) {
                const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(rla, row * 4, 0, 0);
                lar[tb] = Words<4>{{w, w, w, w}};
            }
        }

        // ---- raw tiles, then each thread's own q, k runs (one 4-channel run
        // per owned token) back from them
#pragma unroll
        for (int j = 0; j < VU; ++j) {
            const int u = tid + j * Cfg::NT;
            const int t = u / DU, col = (u % DU) * UE;
            const int pos = bw_pos<Cfg, DM>(t, col);
            lds_store_words(&sm.qh[t][pos], qc[j]);
            lds_store_words(&sm.kh[t][pos], kc[j]);
            lds_store_words(&sm.vv[t][pos], vc[j]);
            lds_store_words(&sm.dout[t][pos], dc[j]);
        }
        __syncthreads();
        Words<RW> qr[TB], kr[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = 16 * tb + r;
            const int pos = bw_pos<Cfg, DM>(t, ch0);
            qr[tb] = *reinterpret_cast<const Words<RW>*>(&sm.qh[t][pos]);
            kr[tb] = *reinterpret_cast<const Words<RW>*>(&sm.kh[t][pos]);
        }

        // the state before the chunk as this wave's dQ operands (bf16: four
        // fragments, in flight through the feature and score stages)
        Frag sfr[BF16 ? D / MK : 1];
        if constexpr (BF16) {
#pragma unroll
            for (int kk = 0; kk < D / MK; ++kk) sfr[kk] = mem_frag<Cfg>(Sc, D, 16 * nb, kk * MK, lane);
        }

        // ---- features, gate prefix and factors of the owned elements.  Only
        // the raw q, k runs and the factor e^{b - r} stay live through the
        // chunk; the features and e^{r - b} are formed again where needed.
        auto feat = [&](const Words<RW>& w, int tb, int i) {
            float a = run_elem<BF16>(w, i);
            if constexpr (ELU1) a = elu1f(a);
            return 16 * tb + r < clen ? a : 0.f;
        };
        float fq[TB][4];
        float er[4];   // e^{r} of the owned channels (DIAG)
#pragma unroll
        for (int i = 0; i < 4; ++i) er[i] = 1.f;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int i = 0; i < 4; ++i) fq[tb][i] = 1.f;
        if constexpr (VG) {
            // inclusive prefix over the chunk's tokens: within each 16-token
            // block across the lanes of a row, then the earlier blocks' totals
            float b[TB][4];
            float carry[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = row_scan16<false>(run_elem<false>(lar[tb], i) * kLog2e);
                    b[tb][i] = x + carry[i];
                    carry[i] += lane_read(x, 16 * g + 15);
                }
            constexpr int tmid = C / 2 - 1;
            float ebr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ref = lane_read(b[tmid / 16][i], 16 * g + tmid % 16);
                const float tot = carry[i];
                er[i] = __builtin_amdgcn_exp2f(ref);
                ebr[i] = __builtin_amdgcn_exp2f(tot - ref);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const float d = b[tb][i] - ref;
                    fq[tb][i] = __builtin_amdgcn_exp2f(d);
                }
            }
            if (r == 0)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    sm.ebr[ch0 + i] = ebr[i];
                    sm.er[ch0 + i] = er[i];
                }
        }

        // ---- Qh, Kh in place of the raw runs
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = 16 * tb + r;
            float x[4], y[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = feat(qr[tb], tb, i) * fq[tb][i];
                y[i] = feat(kr[tb], tb, i) * (VG ? __builtin_amdgcn_rcpf(fq[tb][i]) : 1.f);
            }
            const int pos = bw_pos<Cfg, DM>(t, ch0);
            lds_store_words(&sm.qh[t][pos], pack_run<BF16, 4>(x));
            lds_store_words(&sm.kh[t][pos], pack_run<BF16, 4>(y));
        }
        // the raw runs, opaque from here on, so that the features are
        // formed again from them rather than held through the products
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int j = 0; j < RW; ++j) asm volatile("" : "+v"(qr[tb].w[j]), "+v"(kr[tb].w[j]));
        __syncthreads();

        // ---- P and dP on the lower-triangular tiles, stored transposed
        // [s][t]: the output lane holds four consecutive t of one s
        {
            int idx = 0;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb, ++idx) {
                    if (idx % NW != wave) continue;
                    f32x4_t ap = {0.f, 0.f, 0.f, 0.f}, ad = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < D / MK; ++kk) {
                        ap = T::mma(row_frag<Cfg, DM>(&sm.qh[0][0], D, 16 * tb, kk * MK, lane),
                                    row_frag<Cfg, DM>(&sm.kh[0][0], D, 16 * sb, kk * MK, lane), ap);
                        ad = T::mma(row_frag<Cfg, DM>(&sm.dout[0][0], D, 16 * tb, kk * MK, lane),
                                    row_frag<Cfg, DM>(&sm.vv[0][0], D, 16 * sb, kk * MK, lane), ad);
                    }
                    const int s = 16 * sb + r;
                    float xp[4], xd[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * tb + 4 * g + i;
                        float m = t >= s ? 1.f : 0.f;
                        if constexpr (GATE == LA_GATE_GAMMA) m = t >= s ? sm.gpow[t - s] : 0.f;
                        xp[i] = ap[i] * m;
                        xd[i] = ad[i] * m;
                    }
                    store_run<BF16, 4>(&sm.pt[s][bw_pos<Cfg, TM>(s, 16 * tb + 4 * g)], xp);
                    store_run<BF16, 4>(&sm.dpt[s][bw_pos<Cfg, TM>(s, 16 * tb + 4 * g)], xd);
                }
        }
        __syncthreads();

        // e^{B - r} of G's row 16 nb + r, the row this lane reads
        const float frow = VG ? sm.ebr[16 * nb + r] : 1.f;

        // ---- dQ^T = e^{r} S dO^T + Kh^T dP^T, then * e^{b - r}; with the
        // partial rowsum(Gs * S) of row 16 nb + r (diagonal gate)
        float dqf[TB][4];
        float gss = 0.f;
        {
            f32x4_t acc[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            // (at most 8 steps unrolled: fp32 has 32, whose state loads would
            // all be issued at once)
#pragma unroll 8
            for (int kk = 0; kk < D / MK; ++kk) {
                Frag a;
                if constexpr (BF16) a = sfr[kk];
                else a = mem_frag<Cfg>(Sc, D, 16 * nb, kk * MK, lane);
                if constexpr (VG) {
                    float xs[KPL], xg[KPL];
                    frag_floats<Cfg>(a, xs);
                    g_row<Cfg>(sm.gm, 16 * nb + r, kk * MK + KPL * g, xg);
#pragma unroll
                    for (int j = 0; j < KPL; ++j) gss += xs[j] * xg[j];
                }
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    acc[tb] = T::mma(a, row_frag<Cfg, DM>(&sm.dout[0][0], D, 16 * tb, kk * MK, lane), acc[tb]);
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float f = er[i];
                    if constexpr (GATE == LA_GATE_GAMMA) f = sm.gpow[16 * tb + r + 1];
                    acc[tb][i] *= f;
                }
#pragma unroll
                for (int kk = 0; kk <= (16 * tb + 15) / MK; ++kk)
                    acc[tb] = T::mma(tr_frag<Cfg, DM>(&sm.kh[0][0], D, kk * MK, 16 * nb, lane),
                                     tr_frag<Cfg, TM>(&sm.dpt[0][0], C, kk * MK, 16 * tb, lane), acc[tb]);
#pragma unroll
                for (int i = 0; i < 4; ++i) dqf[tb][i] = acc[tb][i] * fq[tb][i];
            }
        }
        // ---- dK^T = Gs V^T + Qh^T dP, then * e^{r - b}; with the partial
        // sum_s Kh[s][i] (Gs v_s)_i of the chunk's carry (diagonal gate)
        float dkf[TB][4];
        float kgv[4] = {0.f, 0.f, 0.f, 0.f};
        {
            f32x4_t acc[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / MK; ++kk) {
                float xg[KPL];
                g_row<Cfg>(sm.gm, 16 * nb + r, kk * MK + KPL * g, xg);
#pragma unroll
                for (int j = 0; j < KPL; ++j) xg[j] *= frow;
                const Frag a = to_frag<Cfg>(xg);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
                    acc[tb] = T::mma(a, row_frag<Cfg, DM>(&sm.vv[0][0], D, 16 * tb, kk * MK, lane), acc[tb]);
            }
#pragma unroll
            for (int sb = 0; sb < TB; ++sb) {
                if constexpr (VG) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        kgv[i] += acc[sb][i] * (feat(kr[sb], sb, i) * __builtin_amdgcn_rcpf(fq[sb][i]));
                }
                if constexpr (GATE == LA_GATE_GAMMA) {
                    const int s = 16 * sb + r;
                    const float f = s < clen ? sm.gpow[clen - 1 - s] : 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[sb][i] *= f;
                }
#pragma unroll
                for (int kk = (16 * sb) / MK; kk < C / MK; ++kk)
                    acc[sb] = T::mma(tr_frag<Cfg, DM>(&sm.qh[0][0], D, kk * MK, 16 * nb, lane),
                                     row_frag<Cfg, TM>(&sm.dpt[0][0], C, 16 * sb, kk * MK, lane), acc[sb]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dkf[sb][i] = VG ? acc[sb][i] * __builtin_amdgcn_rcpf(fq[sb][i]) : acc[sb][i];
            }
        }
        // ---- dq, dk (chain rule through phi), and db = q dq - k dk for the
        // gate gradient: the features and both gradients end here
        float db[VG ? TB : 1][4];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const uint32_t off = ((uint32_t)(t0 + 16 * tb + r) * D + ch0) * ES;
            float xq[4], xk[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float qf = feat(qr[tb], tb, i), kf = feat(kr[tb], tb, i);
                if constexpr (VG) db[tb][i] = qf * dqf[tb][i] - kf * dkf[tb][i];
                xq[i] = dqf[tb][i];
                xk[i] = dkf[tb][i];
                if constexpr (ELU1) {
                    // phi' = 1 where phi = x + 1 > 1, else phi' = phi = e^x
                    xq[i] *= fminf(qf, 1.f);
                    xk[i] *= fminf(kf, 1.f);
                }
            }
            buf_store_run4<BF16>(rdq, off, xq);
            buf_store_run4<BF16>(rdk, off, xk);
        }
        // ---- dV^T = Gs^T Kh^T + dO^T P
        {
            f32x4_t acc[TB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / MK; ++kk) {
                // Gs's rows kk MK + KPL g + j (the k-slots) in column 16 nb + r
                float xg[KPL];
#pragma unroll
                for (int j = 0; j < KPL; ++j) {
                    const int i = kk * MK + KPL * g + j;
                    xg[j] = sm.gm[g_pos<Cfg>(i, 16 * nb + r)];
                    if constexpr (VG) xg[j] *= sm.ebr[i];
                }
                const Frag a = to_frag<Cfg>(xg);
#pragma unroll
                for (int sb = 0; sb < TB; ++sb)
                    acc[sb] = T::mma(a, row_frag<Cfg, DM>(&sm.kh[0][0], D, 16 * sb, kk * MK, lane), acc[sb]);
            }
#pragma unroll
            for (int sb = 0; sb < TB; ++sb) {
                if constexpr (GATE == LA_GATE_GAMMA) {
                    const int s = 16 * sb + r;
                    const float f = s < clen ? sm.gpow[clen - 1 - s] : 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[sb][i] *= f;
                }
#pragma unroll
                for (int kk = (16 * sb) / MK; kk < C / MK; ++kk)
                    acc[sb] = T::mma(tr_frag<Cfg, DM>(&sm.dout[0][0], D, kk * MK, 16 * nb, lane),
                                     row_frag<Cfg, TM>(&sm.pt[0][0], C, 16 * sb, kk * MK, lane), acc[sb]);
                const uint32_t off = ((uint32_t)(t0 + 16 * sb + r) * D + ch0) * ES;
                float x[4] = {acc[sb][0], acc[sb][1], acc[sb][2], acc[sb][3]};
                buf_store_run4<BF16>(rdv, off, x);
            }
        }

        // ---- G of the chunk before: e^{r} (Gs + Qh^T dO) (diagonal gate),
        // gamma^{clen} G + (q gamma^{t+1})^T dO (gamma), G + Q^T dO, once
        // every wave has read G.  Wave w steps IG row blocks times NG column
        // blocks of G (a 2 x 4 block grid at d = 128, which reads a third
        // less of Qh and dO than whole block rows); the product is formed
        // as dO^T Qh so that the lane holds one row, 4 consecutive columns
        // of each tile.  The product does not involve G and is formed before
        // the barrier; only the read-modify-write of G waits for it.
        constexpr int IG = NW >= 4 ? 2 : 1, NG = NW / IG;
        const int ib0 = (wave % (NW / IG)) * IG, nb0 = (wave / (NW / IG)) * NG;
        f32x4_t gacc[IG][NG];
#pragma unroll
        for (int ii = 0; ii < IG; ++ii)
#pragma unroll
            for (int m = 0; m < NG; ++m) gacc[ii][m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < C / MK; ++kk) {
            Frag bq[IG];
#pragma unroll
            for (int ii = 0; ii < IG; ++ii) {
                bq[ii] = tr_frag<Cfg, DM>(&sm.qh[0][0], D, kk * MK, 16 * (ib0 + ii), lane);
                if constexpr (GATE == LA_GATE_GAMMA) {
                    float x[KPL];
                    frag_floats<Cfg>(bq[ii], x);
#pragma unroll
                    for (int j = 0; j < KPL; ++j) x[j] *= sm.gpow[kk * MK + KPL * g + j + 1];
                    bq[ii] = to_frag<Cfg>(x);
                }
            }
#pragma unroll
            for (int m = 0; m < NG; ++m) {
                const Frag ad = tr_frag<Cfg, DM>(&sm.dout[0][0], D, kk * MK, 16 * (nb0 + m), lane);
#pragma unroll
                for (int ii = 0; ii < IG; ++ii) gacc[ii][m] = T::mma(ad, bq[ii], gacc[ii][m]);
            }
        }

        // ---- the gate gradient
        if constexpr (VG) {
            // the chunk's carry rowsum(G * S_next) per owned channel i:
            //   e^{r_i} rowsum(Gs * S)_i + sum_s Kh[s][i] (Gs v_s)_i
            // the first sum over the four lanes holding row 16 nb + r, read
            // from the lane of each channel; the second over the 16 token lanes
            float rs = gss * frow;
            rs += lane_read(rs, lane ^ 16);
            rs += lane_read(rs, lane ^ 32);
            float later[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float tok = lane_read(row_scan16<false>(kgv[i]), 16 * g + 15);
                later[i] = er[i] * lane_read(rs, 4 * g + i) + tok;
            }
            // suffix sums of db = q dq - k dk over the chunk's tokens: within
            // each block across the lanes, then the later blocks' totals
#pragma unroll
            for (int tb = TB - 1; tb >= 0; --tb) {
                float out[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = row_scan16<true>(db[tb][i]);
                    out[i] = x + later[i];
                    later[i] += lane_read(x, 16 * g);
                }
                if constexpr (GATE == LA_GATE_DIAG) {
                    const uint32_t off = ((uint32_t)(t0 + 16 * tb + r) * D + ch0) * 4;
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4_t, f32x4_t{out[0], out[1], out[2], out[3]}), rdla, off, 0, 0);
                } else {
                    // one gate per token: the sum over all channels, first
                    // over the 4 x 4 channels of this wave's lanes of the token
                    float sum = out[0] + out[1] + out[2] + out[3];
                    sum += lane_read(sum, lane ^ 16);
                    sum += lane_read(sum, lane ^ 32);
                    if (g == 0) sm.red[wave][16 * tb + r] = sum;
                }
            }
            if constexpr (GATE == LA_GATE_SCALAR) {
                // then over the waves
                __syncthreads();
                if (tid < C) {
                    float sum = 0.f;
#pragma unroll
                    for (int w2 = 0; w2 < NW; ++w2) sum += sm.red[w2][tid];
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sum), rdla, (uint32_t)(t0 + tid) * 4, 0, 0);
                }
            }
        }

        __syncthreads();
        {
#pragma unroll
            for (int ii = 0; ii < IG; ++ii) {
                const int gi = 16 * (ib0 + ii) + r;
                // factor on the held G, factor on the sum
                const float fg = GATE == LA_GATE_GAMMA ? sm.gpow[clen] : VG ? sm.ebr[gi] : 1.f;
                const float fo = VG ? sm.er[gi] : 1.f;
#pragma unroll
                for (int m = 0; m < NG; ++m) {
                    float4* pg = reinterpret_cast<float4*>(&sm.gm[g_pos<Cfg>(gi, 16 * (nb0 + m) + 4 * g)]);
                    float4 x = *pg;
                    x.x = fo * (fg * x.x + gacc[ii][m][0]);
                    x.y = fo * (fg * x.y + gacc[ii][m][1]);
                    x.z = fo * (fg * x.z + gacc[ii][m][2]);
                    x.w = fo * (fg * x.w + gacc[ii][m][3]);
                    *pg = x;
                }
            }
        }
        // G stepped; Qh, dO and the factor tables free for the next chunk
        __syncthreads();
    }

    // ---- the gradient of the initial state, from the sequence's first segment
    if (seg == 0 && p.dS0) {
        __syncthreads();
        float4* out = reinterpret_cast<float4*>(p.dS0 + (size_t)bh * D * D);
#pragma unroll
        for (int j = 0; j < GQ; ++j) {
            const int u = tid + j * Cfg::NT;
            out[u] = *reinterpret_cast<const float4*>(&sm.gm[g_pos<Cfg>(u / (D / 4), 4 * (u % (D / 4)))]);
        }
    }
}

// Host-side dispatch over gate mode and feature map for one (d, dtype): one
// workgroup per (b,h) segment.
template <int D, bool BF>
hipError_t launch_bwd_dt(const BwdParams& p, int gate, hipStream_t s) {
    constexpr int C = bwd_chunk(D, BF);
    const dim3 grid((unsigned)(p.BH * p.P));
#define LA_BWD_LAUNCH(GG)                                                                       \
    do {                                                                                        \
        using Cfg = BwdCfg<D, C, BF, GG>;                                                       \
        if (p.phi_elu1)                                                                         \
            LA_LAUNCH((bwd_kernel<Cfg, true>), grid, dim3(Cfg::NT), s, p);          \
        else                                                                                    \
            LA_LAUNCH((bwd_kernel<Cfg, false>), grid, dim3(Cfg::NT), s, p);         \
        return hipGetLastError();                                                               \
    } while (0)
    if (gate == LA_GATE_NONE) LA_BWD_LAUNCH(LA_GATE_NONE);
    if (gate == LA_GATE_GAMMA) LA_BWD_LAUNCH(LA_GATE_GAMMA);
    if (gate == LA_GATE_DIAG) LA_BWD_LAUNCH(LA_GATE_DIAG);
    if (gate == LA_GATE_SCALAR) LA_BWD_LAUNCH(LA_GATE_SCALAR);
    return hipErrorInvalidValue;
#undef LA_BWD_LAUNCH
}

#define LA_DEFINE_BWD_LAUNCHER(NAME, D, BF) \
    hipError_t NAME(const BwdParams& p, int gate, hipStream_t s) { return launch_bwd_dt<D, BF>(p, gate, s); }

}  // namespace la
