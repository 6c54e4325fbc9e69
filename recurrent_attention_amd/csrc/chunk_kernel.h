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
// Matrix-core mapping per chunk (C tokens, d_k x d_v state, fp32 accum):
//   op1  P   = Qh Kh^T        [C x C], lower-triangular 16x16 tiles only
//   op2  O   = Qh S' + P V    [C x d_v]
//   op3  S'' = Kt^T V         [d_k x d_v], accumulated onto the scaled state
// Decay placement by gate mode:
//   NONE  : no scaling.
//   GAMMA : P masked by gamma^(t-s) elementwise (exact for gamma = 0); the
//           Q S term scaled per row by gamma^(t+1); Kt by gamma^(c-1-s);
//           state scaled by gamma^c.  All factors <= 1.
//   DIAG  : factorised around a reference r = b at the chunk middle:
//           Qh = q e^{b_t - r}, Kh = Kt = k e^{r - b_s}; the state is scaled
//           per row by e^{r} before use and by e^{b_{c-1} - r} after the
//           update, so S_new = e^{b_{c-1}-r} (e^{r} S + Kh^T V).
// The state S stays in fp32 matrix-core accumulators for the whole segment;
// wave w owns state columns [w*WN, (w+1)*WN).  For the Q S product the
// accumulators are converted in registers into B operands: lane (n, g) holds
// state rows 16m + 4g + i of column n, so the A operand (Qh) is read with the
// same permutation of the d_k index.
//
// One workgroup runs one (b,h) segment of consecutive chunks.  SONLY = true
// is the state pass: the same loop without q, P and outputs, started from a
// zero state, writing the segment's end state, its decay product and its
// normaliser part to the workspace.
#pragma once

#include "la_device.h"
#include "la_internal.h"

namespace la {

template <int DK_, int DV_, int C_, bool BF16_, int GATE_, bool SONLY_>
struct ChunkCfg {
    static constexpr int DK = DK_, DV = DV_, C = C_, GATE = GATE_;
    static constexpr bool BF16 = BF16_, SONLY = SONLY_;
    using T = Elem<BF16>;
    using E = typename T::E;
    using Pair = typename T::Pair;
    using Frag = typename T::Frag;
    static constexpr int NW = (DV / 16) < 4 ? (DV / 16) : 4;  // waves
    static constexpr int NT = 64 * NW;                         // threads
    static constexpr int WN = DV / NW;                         // state columns per wave
    static constexpr int NB = WN / 16;                         // 16-column blocks per wave
    static constexpr int MB = DK / 16;                         // 16-row blocks of the state
    static constexpr int TB = C / 16;                          // 16-row blocks of a chunk
    static constexpr int KPL = T::KPL, MK = T::MK;
    static constexpr int CP = C < MK ? MK : C;                 // token extent of s-contractions
    // global -> register mapping: each thread owns two adjacent channels
    // (a column pair) over a run of consecutive tokens
    static constexpr int KCP = DK / 2, KTG = NT / KCP, KTPG = C / KTG;
    static constexpr int VCP = DV / 2, VTG = NT / VCP, VTPG = C / VTG;
    static constexpr int PADE = 16 / (int)sizeof(E);           // 16-byte row padding
    static constexpr int QS = DK + PADE;                       // row stride, q/k tiles
    static constexpr int TS = CP + PADE;                       // row stride, transposed tiles and P
    static_assert(DV % 16 == 0 && DK % 16 == 0 && C % 16 == 0, "tile shape");
    static_assert(!BF16 || DK % 32 == 0, "bf16 needs d_k >= 32");
    static_assert(NT % KCP == 0 && NT % VCP == 0, "column-pair mapping");
    static_assert(KTG >= 2 && KTG % 2 == 0 && KTPG >= 1 && VTPG >= 1, "token groups");
    static_assert(KTG * KTPG == C && VTG * VTPG == C, "token groups cover the chunk");
};

template <class Cfg>
struct ChunkSmem {
    using E = typename Cfg::E;
    static constexpr int CQ = Cfg::SONLY ? 1 : Cfg::C;
    alignas(16) E q[CQ][Cfg::QS];     // Qh, row-major [t][i]
    alignas(16) E k[CQ][Cfg::QS];     // Kh, row-major [s][i]
    alignas(16) E kt[Cfg::DK][Cfg::TS];  // Kt, transposed [i][s]
    alignas(16) E vt[Cfg::DV][Cfg::TS];  // V, transposed [n][s]
    alignas(16) E p[CQ][Cfg::TS];     // masked scores [t][s]
    alignas(16) float tot[Cfg::KTG][Cfg::DK];  // per token-group log-gate sums
    float pre[Cfg::DK], post[Cfg::DK];
    float gpow[Cfg::C + 2];           // gamma^j
    float z[Cfg::DK];
    float den[Cfg::C];
};

template <class Cfg>
__device__ __forceinline__ void scale_rows(f32x4_t (&acc)[Cfg::MB][Cfg::NB], const float* f, int g) {
#pragma unroll
    for (int mb = 0; mb < Cfg::MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = f[16 * mb + 4 * g + i];
#pragma unroll
            for (int nb = 0; nb < Cfg::NB; ++nb) acc[mb][nb][i] *= s;
        }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void chunk_kernel(const ChunkParams p) {
    constexpr int DK = Cfg::DK, DV = Cfg::DV, C = Cfg::C, GATE = Cfg::GATE;
    constexpr int NB = Cfg::NB, MB = Cfg::MB, TB = Cfg::TB, NW = Cfg::NW;
    constexpr int KPL = Cfg::KPL, MK = Cfg::MK, CP = Cfg::CP;
    constexpr int KCP = Cfg::KCP, KTG = Cfg::KTG, KTPG = Cfg::KTPG;
    constexpr int VCP = Cfg::VCP, VTPG = Cfg::VTPG;
    constexpr bool SONLY = Cfg::SONLY, BF16 = Cfg::BF16;
    using T = typename Cfg::T;
    using E = typename Cfg::E;
    using Pair = typename Cfg::Pair;
    using Frag = typename Cfg::Frag;

    __shared__ ChunkSmem<Cfg> sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int P = p.P;
    const int PS = SONLY ? P - 1 : P;  // the state pass skips the last segment
    const int seg = blockIdx.x % PS;
    const int bh = blockIdx.x / PS;
    const int h = bh % p.H;
    const int L = p.L;
    const int c_begin = seg * p.cps;
    const int c_end = min(c_begin + p.cps, p.nchunks);
    const int elu1 = p.phi_elu1;
    const bool norm = p.normalize != 0;

    const int kcp = tid % KCP, ktg = tid / KCP;
    const int vcp = tid % VCP, vtg = tid / VCP;
    const int colbase = wave * Cfg::WN;

    // ---- one-time LDS set-up: zero the tiles whose padding is read as zeros
    {
        E* z0p = &sm.kt[0][0];
        for (int i = tid; i < DK * Cfg::TS; i += Cfg::NT) z0p[i] = E(0);
        E* z1p = &sm.vt[0][0];
        for (int i = tid; i < DV * Cfg::TS; i += Cfg::NT) z1p[i] = E(0);
        if constexpr (!SONLY) {
            E* z2p = &sm.p[0][0];
            for (int i = tid; i < C * Cfg::TS; i += Cfg::NT) z2p[i] = E(0);
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
    if constexpr (!SONLY) {
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

    // segment decay product (state pass)
    float seg_la = 0.0f, seg_lb = 0.0f;  // DIAG: summed log-gates of this thread's channels
    float seg_g = 1.0f;                  // GAMMA: product of gamma^c

    // ---- register prefetch of one chunk
    const Pair* qp = reinterpret_cast<const Pair*>(p.q);
    const Pair* kp = reinterpret_cast<const Pair*>(p.k);
    const Pair* vp = reinterpret_cast<const Pair*>(p.v);
    const float2* lap = reinterpret_cast<const float2*>(p.log_alpha);
    Pair rq[KTPG], rk[KTPG], rv[VTPG];
    float2 rla[KTPG];
    auto load_chunk = [&](int c) {
        const int t0 = c * C;
#pragma unroll
        for (int j = 0; j < KTPG; ++j) {
            const int t = t0 + ktg * KTPG + j;
            const bool ok = t < L;
            const size_t off = ((size_t)bh * L + t) * (DK / 2) + kcp;
            if constexpr (!SONLY) rq[j] = ok ? qp[off] : T::zero();
            rk[j] = ok ? kp[off] : T::zero();
            if constexpr (GATE == LA_GATE_DIAG) rla[j] = ok ? lap[off] : make_float2(0.f, 0.f);
        }
#pragma unroll
        for (int j = 0; j < VTPG; ++j) {
            const int t = t0 + vtg * VTPG + j;
            const bool ok = t < L;
            const size_t off = ((size_t)bh * L + t) * (DV / 2) + vcp;
            rv[j] = ok ? vp[off] : T::zero();
        }
    };
    if (c_begin < c_end) load_chunk(c_begin);

    for (int c = c_begin; c < c_end; ++c) {
        const int t0 = c * C;
        const int clen = min(C, L - t0);

        // ---- a1: features; a2: chunk-local inclusive log-gate prefix
        float qa[KTPG], qb[KTPG], ka[KTPG], kb[KTPG], ba[KTPG], bb[KTPG];
        {
            float ca = 0.f, cb = 0.f;
#pragma unroll
            for (int j = 0; j < KTPG; ++j) {
                const bool ok = (ktg * KTPG + j) < clen;
                ka[j] = ok ? feature(T::lo(rk[j]), elu1) : 0.f;
                kb[j] = ok ? feature(T::hi(rk[j]), elu1) : 0.f;
                if constexpr (!SONLY) {
                    qa[j] = feature(T::lo(rq[j]), elu1);
                    qb[j] = feature(T::hi(rq[j]), elu1);
                }
                if constexpr (GATE == LA_GATE_DIAG) {
                    ca += rla[j].x;
                    cb += rla[j].y;
                    ba[j] = ca;
                    bb[j] = cb;
                }
            }
            if constexpr (GATE == LA_GATE_DIAG) {
                __syncthreads();  // the previous chunk is done with every LDS tile
                sm.tot[ktg][2 * kcp] = ca;
                sm.tot[ktg][2 * kcp + 1] = cb;
            }
        }
        // NONE/GAMMA: the previous chunk is done with every LDS tile.
        // DIAG: the token-group sums are visible.
        __syncthreads();

        float refa = 0.f, refb = 0.f, tota = 0.f, totb = 0.f, offa = 0.f, offb = 0.f;
        if constexpr (GATE == LA_GATE_DIAG) {
#pragma unroll
            for (int g2 = 0; g2 < KTG; ++g2) {
                const float2 tv = *reinterpret_cast<const float2*>(&sm.tot[g2][2 * kcp]);
                if (g2 < ktg) { offa += tv.x; offb += tv.y; }
                if (g2 < KTG / 2) { refa += tv.x; refb += tv.y; }
                tota += tv.x;
                totb += tv.y;
            }
            seg_la += tota;
            seg_lb += totb;
        }
        if constexpr (GATE == LA_GATE_GAMMA) seg_g *= sm.gpow[clen];

        // ---- write the chunk's tiles to LDS
        {
            float kta[KTPG], ktb[KTPG];
#pragma unroll
            for (int j = 0; j < KTPG; ++j) {
                const int t = ktg * KTPG + j;
                float fqa = 1.f, fqb = 1.f, fka = 1.f, fkb = 1.f, fta = 1.f, ftb = 1.f;
                if constexpr (GATE == LA_GATE_DIAG) {
                    const float bta = offa + ba[j], btb = offb + bb[j];
                    fqa = __expf(bta - refa);
                    fqb = __expf(btb - refb);
                    fka = __expf(refa - bta);
                    fkb = __expf(refb - btb);
                    fta = fka;
                    ftb = fkb;
                } else if constexpr (GATE == LA_GATE_GAMMA) {
                    fta = ftb = t < clen ? sm.gpow[clen - 1 - t] : 0.f;
                }
                if constexpr (!SONLY) {
                    *reinterpret_cast<Pair*>(&sm.q[t][2 * kcp]) = T::pack(qa[j] * fqa, qb[j] * fqb);
                    *reinterpret_cast<Pair*>(&sm.k[t][2 * kcp]) = T::pack(ka[j] * fka, kb[j] * fkb);
                }
                kta[j] = ka[j] * fta;
                ktb[j] = kb[j] * ftb;
            }
            store_run<BF16, KTPG>(&sm.kt[2 * kcp][ktg * KTPG], kta);
            store_run<BF16, KTPG>(&sm.kt[2 * kcp + 1][ktg * KTPG], ktb);
            float va[VTPG], vb[VTPG];
#pragma unroll
            for (int j = 0; j < VTPG; ++j) {
                va[j] = T::lo(rv[j]);
                vb[j] = T::hi(rv[j]);
            }
            store_run<BF16, VTPG>(&sm.vt[2 * vcp][vtg * VTPG], va);
            store_run<BF16, VTPG>(&sm.vt[2 * vcp + 1][vtg * VTPG], vb);
            if (ktg == 0) {
                float prea = 1.f, preb = 1.f, posta = 1.f, postb = 1.f;
                if constexpr (GATE == LA_GATE_DIAG) {
                    prea = __expf(refa);
                    preb = __expf(refb);
                    posta = __expf(tota - refa);
                    postb = __expf(totb - refb);
                } else if constexpr (GATE == LA_GATE_GAMMA) {
                    prea = preb = sm.gpow[clen];
                }
                sm.pre[2 * kcp] = prea;
                sm.pre[2 * kcp + 1] = preb;
                sm.post[2 * kcp] = posta;
                sm.post[2 * kcp + 1] = postb;
            }
        }

        // ---- prefetch the next chunk while this one is computed
        if (c + 1 < c_end) load_chunk(c + 1);
        __syncthreads();

        // ---- op1: masked in-chunk scores, lower-triangular tiles
        if constexpr (!SONLY) {
            int idx = 0;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb, ++idx) {
                    if (idx % NW != wave) continue;
                    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < DK / MK; ++kk) {
                        const Frag a = T::load(&sm.q[16 * tb + r][kk * MK + KPL * g]);
                        const Frag b = T::load(&sm.k[16 * sb + r][kk * MK + KPL * g]);
                        acc = T::mma(a, b, acc);
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * tb + 4 * g + i, s = 16 * sb + r;
                        float val = acc[i];
                        if (s > t) val = 0.f;
                        else if constexpr (GATE == LA_GATE_GAMMA) val *= sm.gpow[t - s];
                        sm.p[t][s] = T::fromf(val);
                    }
                }
            }
            __syncthreads();

            // ---- a4: normaliser of each row, read with the state before this chunk
            if (norm) {
                if (tid < C) {
                    const int t = tid;
                    float rs = 0.f;
                    for (int s = 0; s <= t; ++s) rs += T::tof(sm.p[t][s]);
                    float dq = 0.f;
                    for (int i = 0; i < DK; ++i) {
                        float zz = sm.z[i];
                        if constexpr (GATE == LA_GATE_DIAG) zz *= sm.pre[i];
                        dq += T::tof(sm.q[t][i]) * zz;
                    }
                    if constexpr (GATE == LA_GATE_GAMMA) dq *= sm.gpow[t + 1];
                    sm.den[t] = dq + rs;
                }
                __syncthreads();
            }
        }
        // z <- post * (pre * z + sum_s Kt[:, s])  (each thread its own channel)
        if (norm && tid < DK) {
            float cs = 0.f;
            for (int s = 0; s < C; ++s) cs += T::tof(sm.kt[tid][s]);
            sm.z[tid] = sm.post[tid] * (sm.pre[tid] * sm.z[tid] + cs);
        }

        // ---- value fragments, shared by op2 and op3
        Frag vf[CP / MK][NB];
#pragma unroll
        for (int kk = 0; kk < CP / MK; ++kk)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
                vf[kk][nb] = T::load(&sm.vt[colbase + 16 * nb + r][kk * MK + KPL * g]);

        if constexpr (GATE == LA_GATE_DIAG) scale_rows<Cfg>(accS, sm.pre, g);

        if constexpr (!SONLY) {
            // ---- op2: O = Qh S' (+ row decay) + P V
            f32x4_t accO[TB][NB];
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) accO[tb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            if constexpr (BF16) {
#pragma unroll
                for (int k2 = 0; k2 < DK / 32; ++k2) {
                    Frag bs[NB];
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const float x[8] = {accS[2 * k2][nb][0], accS[2 * k2][nb][1],
                                            accS[2 * k2][nb][2], accS[2 * k2][nb][3],
                                            accS[2 * k2 + 1][nb][0], accS[2 * k2 + 1][nb][1],
                                            accS[2 * k2 + 1][nb][2], accS[2 * k2 + 1][nb][3]};
                        bs[nb] = T::from8(x);
                    }
#pragma unroll
                    for (int tb = 0; tb < TB; ++tb) {
                        const Frag a = T::load2x4(&sm.q[16 * tb + r][32 * k2 + 4 * g],
                                                  &sm.q[16 * tb + r][32 * k2 + 16 + 4 * g]);
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) accO[tb][nb] = T::mma(a, bs[nb], accO[tb][nb]);
                    }
                }
            } else {
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int tb = 0; tb < TB; ++tb) {
                            const Frag a = sm.q[16 * tb + r][16 * mb + 4 * g + i];
#pragma unroll
                            for (int nb = 0; nb < NB; ++nb)
                                accO[tb][nb] = T::mma(a, accS[mb][nb][i], accO[tb][nb]);
                        }
            }
            if constexpr (GATE == LA_GATE_GAMMA) {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float f = sm.gpow[16 * tb + 4 * g + i + 1];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) accO[tb][nb][i] *= f;
                    }
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
                for (int kk = 0; kk <= (16 * tb + 15) / MK; ++kk) {
                    const Frag a = T::load(&sm.p[16 * tb + r][kk * MK + KPL * g]);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) accO[tb][nb] = T::mma(a, vf[kk][nb], accO[tb][nb]);
                }
            }
            // ---- store the chunk's outputs
            E* outp = reinterpret_cast<E*>(p.out);
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * tb + 4 * g + i;
                    if (t < clen) {
                        const float inv = norm ? 1.0f / sm.den[t] : 1.0f;
                        E* row = outp + ((size_t)bh * L + t0 + t) * DV + colbase + r;
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb) row[16 * nb] = T::fromf(accO[tb][nb][i] * inv);
                    }
                }
        }

        // ---- op3: state update
        if constexpr (GATE == LA_GATE_GAMMA) scale_rows<Cfg>(accS, sm.pre, g);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int kk = 0; kk < CP / MK; ++kk) {
                const Frag a = T::load(&sm.kt[16 * mb + r][kk * MK + KPL * g]);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) accS[mb][nb] = T::mma(a, vf[kk][nb], accS[mb][nb]);
            }
        if constexpr (GATE == LA_GATE_DIAG) scale_rows<Cfg>(accS, sm.post, g);
    }

    // ---- epilogue
    float* Sout;
    float* zout;
    if constexpr (SONLY) {
        Sout = p.ws_S + ((size_t)bh * P + seg) * SS;
        zout = p.ws_z + ((size_t)bh * P + seg) * DK;
        float* aout = p.ws_a + ((size_t)bh * P + seg) * DK;
        if constexpr (GATE == LA_GATE_DIAG) {
            if (ktg == 0) {
                aout[2 * kcp] = __expf(seg_la);
                aout[2 * kcp + 1] = __expf(seg_lb);
            }
        } else {
            if (tid < DK) aout[tid] = GATE == LA_GATE_GAMMA ? seg_g : 1.0f;
        }
    } else {
        if (seg != P - 1) return;
        Sout = p.S_final;
        zout = p.z_final;
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
template <int DK, int DV>
__global__ __launch_bounds__(256) void state_scan_kernel(const ChunkParams p) {
    constexpr int N4 = DK * DV / 4;
    constexpr int NBX = (N4 + 255) / 256;
    const int bh = blockIdx.x / NBX;
    const int bx = blockIdx.x % NBX;
    const int e4 = bx * 256 + threadIdx.x;
    const int P = p.P;
    const size_t SS = (size_t)DK * DV;
    if (e4 < N4) {
        const int row = (e4 * 4) / DV;
        float4 x = p.S0 ? reinterpret_cast<const float4*>(p.S0 + (size_t)bh * SS)[e4]
                        : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < P - 1; ++j) {
            float4* slot = reinterpret_cast<float4*>(p.ws_S + ((size_t)bh * P + j) * SS) + e4;
            const float4 u = *slot;
            *slot = x;
            const float a = p.ws_a[((size_t)bh * P + j) * DK + row];
            x = make_float4(a * x.x + u.x, a * x.y + u.y, a * x.z + u.z, a * x.w + u.w);
        }
        reinterpret_cast<float4*>(p.ws_S + ((size_t)bh * P + P - 1) * SS)[e4] = x;
    }
    if (p.normalize && bx == 0 && threadIdx.x < DK) {
        const int i = threadIdx.x;
        float zx = p.z0 ? p.z0[(size_t)bh * DK + i] : 0.f;
        for (int j = 0; j < P - 1; ++j) {
            float* slot = p.ws_z + ((size_t)bh * P + j) * DK + i;
            const float u = *slot;
            *slot = zx;
            zx = p.ws_a[((size_t)bh * P + j) * DK + i] * zx + u;
        }
        p.ws_z[((size_t)bh * P + P - 1) * DK + i] = zx;
    }
}

// Host-side dispatch over chunk length and gate mode for one (d, dtype).
template <int D, bool BF>
hipError_t launch_chunk_dt(const ChunkParams& p, int chunk, int gate, bool sonly, hipStream_t s,
                           int nblocks) {
#define LA_CHUNK_LAUNCH(CC, GG, SO)                                                      \
    do {                                                                                 \
        using Cfg = ChunkCfg<D, D, CC, BF, GG, SO>;                                      \
        hipLaunchKernelGGL((chunk_kernel<Cfg>), dim3(nblocks), dim3(Cfg::NT), 0, s, p);  \
        return hipGetLastError();                                                        \
    } while (0)
#define LA_CHUNK_GATES(CC, SO)                                   \
    do {                                                         \
        if (gate == LA_GATE_NONE) LA_CHUNK_LAUNCH(CC, 0, SO);    \
        if (gate == LA_GATE_GAMMA) LA_CHUNK_LAUNCH(CC, 1, SO);   \
        LA_CHUNK_LAUNCH(CC, 2, SO);                              \
    } while (0)
#define LA_CHUNK_SONLY(CC)                             \
    do {                                               \
        if (sonly) LA_CHUNK_GATES(CC, true);           \
        LA_CHUNK_GATES(CC, false);                     \
    } while (0)
    if (chunk == 16) LA_CHUNK_SONLY(16);
    if (chunk == 32) LA_CHUNK_SONLY(32);
    if (chunk == 64) LA_CHUNK_SONLY(64);
    return hipErrorInvalidValue;
#undef LA_CHUNK_SONLY
#undef LA_CHUNK_GATES
#undef LA_CHUNK_LAUNCH
}

// One explicit (d, dtype) instantiation per translation unit.
#define LA_DEFINE_CHUNK_LAUNCHER(NAME, D, BF)                                                      \
    hipError_t NAME(const ChunkParams& p, int chunk, int gate, bool sonly, hipStream_t s,          \
                    int nblocks) {                                                                 \
        return launch_chunk_dt<D, BF>(p, chunk, gate, sonly, s, nblocks);                          \
    }

}  // namespace la
