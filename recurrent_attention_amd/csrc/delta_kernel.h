// delta_kernel.h -- the delta rule (DeltaNet recurrence of
// "linear_sparse_attention.py", function delta_rule_recurrent) on gfx950:
//
//   S_t = (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = q_t^T S_t
//
// in the [d_k][d_v] state orientation of the rest of the library (the page
// writes the transpose).  Keys are used as given.
//
// Prefill, chunkwise (the pages give the recurrence only; this is the
// standard triangular factorisation of the product of the chunk's erase
// matrices, restated): for a chunk of C tokens with state S before it,
//   A  = strict_lower(diag(beta) K K^T),  T = (I + A)^-1 diag(beta)
//   U' = T (V - K S)
//   O  = Q S + (Q K^T * inclusive causal mask) U',   S <- S + K^T U'
// because the chunk's product of (I - beta k k^T) factors is I - K^T W and
// its accumulated writes are K^T U, with W = T K and U = T V (so that
// U' = U - W S; W itself is never formed).  Everything but T is a dense
// product on the matrix cores; T is formed by blocked forward substitution
// (16 x 16 diagonal blocks inverted in fp32 by one or two lanes per column,
// the blocks below them by matrix-core products, bf16 operands with fp32
// sums for bf16 inputs and fp32 throughout for fp32 inputs, one block
// column per wave).
//
// One workgroup per (b,h) runs the chunks in order (the chunk-to-chunk map
// S -> (I - K^T W) S + K^T U is a full d_k x d_k matrix, so the segment
// split of the gated kernels does not carry over cheaply).  Wave w owns
// value columns [16w, 16w+16): its state block stays in fp32 accumulators
// and it produces those columns of V - K S, U' and the outputs, all three
// in registers (a matrix-core result becomes the next product's operand
// with its token index permuted, the other operand read to match).
//
// Decode: one workgroup per (b,h) streams its fp32 state once:
//   u = S^T k, w = S^T q (one reduction pass), S += beta k (v - u)^T,
//   o = w + beta (q . k) (v - u).
#pragma once

#include "la_device.h"
#include "la_internal.h"
#include "tile_ops.h"

namespace la {

template <int D_, int C_, bool BF16_>
struct DeltaCfg {
    static constexpr int D = D_, C = C_;
    static constexpr bool BF16 = BF16_;
    using T = Elem<BF16>;
    using E = typename T::E;
    using Frag = typename T::Frag;
    static constexpr int NW = D / 16;                  // waves: one value block each
    static constexpr int NT = 64 * NW;
    static constexpr int TB = C / 16, NBLK = C / 16, MB = D / 16;
    static constexpr int KPL = T::KPL, MK = T::MK;
    static constexpr int UE = 16 / (int)sizeof(E);
    static constexpr int DU = D / UE, TU = C / UE;
    // the D-wide tiles swizzle over up to 16 units (256 bytes): the LDS has
    // 64 four-byte banks, so 16 consecutive rows of a fragment read fall on
    // 16 different bank groups
    static constexpr int DMASK = (DU < 16 ? DU : 16) - 1;
    static constexpr int TMASK = (TU < 8 ? TU : 8) - 1;
    static constexpr int CPR = 16 / (int)sizeof(E);   // channels of a 16-byte run
    static constexpr int RUNS = D / CPR;               // runs per token row
    static constexpr int RPP = NT / RUNS;              // token rows per load pass
    static constexpr int NPASS = C / RPP;
    static constexpr int RW = 4;                       // words of a run
    static_assert(D % 16 == 0 && C % 16 == 0 && C % MK == 0, "tile shape");
    static_assert(!BF16 || D % 32 == 0, "bf16 needs d >= 32");
    static_assert(NT % RUNS == 0 && C % RPP == 0, "load mapping");
};

template <class Cfg>
struct DeltaSmem {
    using E = typename Cfg::E;
    static constexpr int C = Cfg::C, D = Cfg::D;
    alignas(16) E q[C][D];        // Q   [t][swizzled i]
    alignas(16) E k[C][D];        // K   [s][swizzled i]
    alignas(16) E v[C][D];        // V   [s][swizzled n]
    alignas(16) E pm[C][C];       // P = Q K^T * mask  [t][swizzled s]
    alignas(16) E tm[C][C];       // T   [s][swizzled j]
    // A (strictly lower) and the diagonal blocks of N = (I + A)^-1 in fp32,
    // rows padded by 4 so that 16 lanes reading one column of 16 rows spread
    // over the banks (only those blocks are ever used)
    static constexpr int LDP = C + 4;
    alignas(16) float lm[C][LDP];
    alignas(16) float nm[C][LDP];
    // with 8 waves over 64-token chunks, wave 0's state block as operand
    // fragments (lane-major) and the S^T Q^T that wave 3 forms from them
    static constexpr bool HELP = Cfg::BF16 && Cfg::NW == 8 && Cfg::NBLK == 4;
    alignas(16) uint4 sa0[HELP ? D / 32 : 1][64];
    alignas(16) f32x4_t oq0[HELP ? Cfg::TB : 1][64];
    float beta[C];
};

// Position of column `col` in row `row` of the C x C tiles (P and T).  Their
// bf16 rows of 128 bytes XOR the unit index with row ^ (row >> 3): the tiles
// are read in 8-byte row reads (16 rows, two half-units each, per pass of 32
// lanes), which the plain row index leaves two-way conflicted (rows 8 apart
// share their banks).
template <class Cfg>
__device__ __forceinline__ int cc_pos(int row, int col) {
    if constexpr (Cfg::BF16 && Cfg::C == 64) {
        const int u = col / Cfg::UE, e = col % Cfg::UE;
        return ((u ^ ((row ^ (row >> 3)) & 7)) * Cfg::UE) + e;
    } else {
        return bw_pos<Cfg, Cfg::TMASK>(row, col);
    }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT) void delta_chunk_kernel(const DeltaParams p) {
    constexpr int D = Cfg::D, C = Cfg::C, TB = Cfg::TB, NW = Cfg::NW, NBLK = Cfg::NBLK;
    constexpr int MB = Cfg::MB, MK = Cfg::MK, KPL = Cfg::KPL, RW = Cfg::RW;
    constexpr int RUNS = Cfg::RUNS, NPASS = Cfg::NPASS, RPP = Cfg::RPP;
    constexpr int DM = Cfg::DMASK;
    constexpr bool BF16 = Cfg::BF16;
    constexpr int ES = (int)sizeof(typename Cfg::E);
    using T = typename Cfg::T;
    using F = Elem<false>;   // fp32 matrix cores for the triangular solve
    using E = typename Cfg::E;
    using Frag = typename Cfg::Frag;

    __shared__ DeltaSmem<Cfg> sm;
    auto& lm = sm.lm;
    auto& nm = sm.nm;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int r = lane & 15, g = lane >> 4;
    const int bh = blockIdx.x;
    const int L = p.L;
    const int nchunks = (L + C - 1) / C;
    const int n0 = 16 * wave;   // this wave's value columns

    const size_t rows0 = (size_t)bh * L;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(reinterpret_cast<const E*>(p.q) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(reinterpret_cast<const E*>(p.k) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(reinterpret_cast<const E*>(p.v) + rows0 * D, (uint32_t)L * D * ES);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.beta + rows0, (uint32_t)L * 4);
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(reinterpret_cast<E*>(p.out) + rows0 * D, (uint32_t)L * D * ES);

    // the triangular tiles: only their lower parts are ever written (the
    // blocks of A and N that are used are written in full in every chunk,
    // and nothing reads the rest)
    for (int i = tid; i < C * C; i += Cfg::NT) {
        (&sm.pm[0][0])[i] = E(0);
        (&sm.tm[0][0])[i] = E(0);
    }

    // state block of this wave: rows 16 mb + 4 g + i, column n0 + r
    f32x4_t accS[MB];
    const float* S0 = p.S0 ? p.S0 + (size_t)bh * D * D : nullptr;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            accS[mb][i] = S0 ? S0[(size_t)(16 * mb + 4 * g + i) * D + n0 + r] : 0.f;

    // global -> registers, one chunk ahead: a 16-byte run of q, k, v for
    // NPASS token rows, and one write strength (non-temporal loads: each
    // element is read once)
    const int run = tid % RUNS, row0 = tid / RUNS;
    Words<RW> qr[NPASS], kr[NPASS], vr[NPASS];
    uint32_t br = 0;
    auto load = [&](int c) {
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            const uint32_t off = (((uint32_t)c * C + row0 + RPP * ps) * D + Cfg::CPR * run) * ES;
            qr[ps] = buf_load_words<RW, LOAD_NT>(rq, off);
            kr[ps] = buf_load_words<RW, LOAD_NT>(rk, off);
            vr[ps] = buf_load_words<RW, LOAD_NT>(rv, off);
        }
        if (tid < C) br = __builtin_amdgcn_raw_buffer_load_b32(rb, ((uint32_t)c * C + tid) * 4, 0, LOAD_NT);
    };
    if (nchunks > 0) load(0);

    for (int c = 0; c < nchunks; ++c) {
        // the lane index, opaque to the compiler in each chunk: otherwise the
        // many lane-dependent LDS addresses of a chunk are hoisted out of the
        // walk and held in registers across it; masked again, so that the
        // compiler still knows its range (a lane index it must take as
        // possibly negative turns every column / 8 of the tile addresses
        // into a signed division)
        int lane_o = tid & 63;
        asm volatile("" : "+v"(lane_o));
        const int lane = lane_o & 63;
        const int r = lane & 15, g = lane >> 4;
        const int t0 = c * C;
        // ---- tiles (tokens past the end read as zeros: no key, no write)
#pragma unroll
        for (int ps = 0; ps < NPASS; ++ps) {
            const int t = row0 + RPP * ps;
            const int pos = bw_pos<Cfg, DM>(t, Cfg::CPR * run);
            lds_store_words(&sm.q[t][pos], qr[ps]);
            lds_store_words(&sm.k[t][pos], kr[ps]);
            lds_store_words(&sm.v[t][pos], vr[ps]);
        }
        if (tid < C) sm.beta[tid] = __uint_as_float(br);
        __syncthreads();

        // ---- the state as an operand: rows n of S^T (or columns n of S),
        // k-slots the state rows held by this lane (32 k2 + 4 g + i and
        // 32 k2 + 16 + 4 g + i)
        Frag sa[BF16 ? D / 32 : 1];
        if constexpr (BF16) {
#pragma unroll
            for (int k2 = 0; k2 < D / 32; ++k2) {
                const float x8[8] = {accS[2 * k2][0], accS[2 * k2][1], accS[2 * k2][2], accS[2 * k2][3],
                                     accS[2 * k2 + 1][0], accS[2 * k2 + 1][1], accS[2 * k2 + 1][2],
                                     accS[2 * k2 + 1][3]};
                sa[k2] = T::from8(x8);
            }
        }
        // wave 0 lends its state block to the helper wave (read after the
        // barrier that ends the diagonal solve, rewritten only after the
        // next chunk's first barrier)
        constexpr bool HELP = DeltaSmem<Cfg>::HELP;
        constexpr int HW = 3;   // the helper: no block column, SIMD shared with wave 7
        if constexpr (HELP) {
            if (wave == 0)
#pragma unroll
                for (int k2 = 0; k2 < D / 32; ++k2) sm.sa0[k2][lane] = __builtin_bit_cast(uint4, sa[k2]);
        }
        // the rows s = 16 xb + r of a D-wide tile X, k-slots matching sa
        auto x_frag = [&](const E* X, int xb, int k2) -> Frag {
            if constexpr (BF16) {
                const int s = 16 * xb + r;
                return T::load2x4(X + s * D + bw_pos<Cfg, DM>(s, 32 * k2 + 4 * g),
                                  X + s * D + bw_pos<Cfg, DM>(s, 32 * k2 + 16 + 4 * g));
            } else {
                return Frag{};
            }
        };
        // S^T X^T for the rows s (or t) = 16 xb + r of tile X: lane slot i
        // holds value column n0 + 4 g + i
        auto state_times = [&](const E* X, int xb, f32x4_t acc) {
            if constexpr (BF16) {
#pragma unroll
                for (int k2 = 0; k2 < D / 32; ++k2) acc = T::mma(sa[k2], x_frag(X, xb, k2), acc);
            } else {
                const int s = 16 * xb + r;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = T::mma(accS[mb][i], X[s * D + bw_pos<Cfg, DM>(s, 16 * mb + 4 * g + i)], acc);
            }
            return acc;
        };
        // X S for the rows 16 xb + 4 g + i of tile X (lane slot i) and this
        // lane's value column n0 + r: the same reads, operands swapped
        auto times_state = [&](const E* X, int xb, f32x4_t acc) {
            if constexpr (BF16) {
#pragma unroll
                for (int k2 = 0; k2 < D / 32; ++k2) acc = T::mma(x_frag(X, xb, k2), sa[k2], acc);
            } else {
                const int s = 16 * xb + r;
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = T::mma(X[s * D + bw_pos<Cfg, DM>(s, 16 * mb + 4 * g + i)], accS[mb][i], acc);
            }
            return acc;
        };
        // V - K S for this wave's value columns, tokens 16 xb + 4 g + i of
        // lane slot i (V read transposed into that layout)
        f32x4_t xt[TB];
        auto form_xt = [&]() {
#pragma unroll
            for (int xb = 0; xb < TB; ++xb) {
                f32x4_t vx;
                if constexpr (BF16) {
                    const int row = 16 * xb + 4 * g + (r >> 2);
                    const auto* pv = &sm.v[row][bw_pos<Cfg, DM>(row, n0 + 4 * (r & 3))];
                    const bw_i16x4 t4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) bw_i16x4*)(pv));
                    const uint2 u = __builtin_bit_cast(uint2, t4);
                    vx = f32x4_t{-bf16lo(u.x), -bf16hi(u.x), -bf16lo(u.y), -bf16hi(u.y)};
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * xb + 4 * g + i;
                        vx[i] = -sm.v[row][bw_pos<Cfg, DM>(row, n0 + r)];
                    }
                }
                xt[xb] = -times_state(&sm.k[0][0], xb, vx);
            }
        };

        // ---- A = strict_lower(diag(beta) K K^T), computed transposed ([s][t]
        // tiles) so each lane holds 4 consecutive s of one t
        {
            int idx = 0;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb, ++idx) {
                    if (idx % NW != wave) continue;
                    f32x4_t ag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kk = 0; kk < D / MK; ++kk)
                        ag = T::mma(row_frag<Cfg, DM>(&sm.k[0][0], D, 16 * sb, kk * MK, lane),
                                    row_frag<Cfg, DM>(&sm.k[0][0], D, 16 * tb, kk * MK, lane), ag);
                    const int t = 16 * tb + r, s0 = 16 * sb + 4 * g;
                    const float bt = sm.beta[t];
                    float xl[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) xl[i] = s0 + i < t ? bt * ag[i] : 0.f;
                    *reinterpret_cast<float4*>(&lm[t][s0]) = make_float4(xl[0], xl[1], xl[2], xl[3]);
                }
        }
        __syncthreads();

        // ---- the diagonal 16 x 16 blocks of N = (I + A)^-1 by forward
        // substitution in wave 0, one lane per column (lane 16 blk + j solves
        // column j of block blk: no exchange between lanes, A's rows read as
        // broadcasts); their part of T = N diag(beta) with them.  The other
        // waves meanwhile form P = Q K^T * inclusive mask ([s][t] tiles, as
        // for A).  Then every wave forms its columns of V - K S, which needs
        // only the state, K and V.
        {
            // with 8 waves: two lanes per column on waves 0 and 1 (two blocks
            // each), each lane summing half of every row's terms
            constexpr bool SOLVE2 = NW == 8;
            if (SOLVE2 ? wave < 2 : wave == 0) {
                if constexpr (SOLVE2) {
                    // lane 32 bs + 2 j + h solves column j of block 2 w + bs; it
                    // keeps the rows of the groups of four 4 h.. and 8 + 4 h..
                    // (slot p: row 8 (p >> 2) + 4 h + (p & 3)) and sums their
                    // terms (terms of rows not yet solved are zero: their A
                    // entries are on or above the diagonal); one DPP swap
                    // adds the partner lane's half
                    const int bs = lane >> 5, j = (lane >> 1) & 15, h = lane & 1;
                    const int blk = 2 * wave + bs;
                    if (blk < NBLK) {
                        const int b0 = 16 * blk;
                        float xs[8];
#pragma unroll
                        for (int q = 0; q < 8; ++q) xs[q] = 0.f;
                        float4 arow[16][2];
                        auto read_row = [&](int rr) {
#pragma unroll
                            for (int q = 0; 8 * q < rr; ++q)
                                arow[rr][q] = *reinterpret_cast<const float4*>(&lm[b0 + rr][b0 + 8 * q + 4 * h]);
                        };
                        read_row(1);
                        read_row(2);
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            if (rr + 2 < 16) read_row(rr + 2);
                            float part[2] = {0.f, 0.f};
#pragma unroll
                            for (int q = 0; 8 * q < rr; ++q)
                                part[q] = (arow[rr][q].x * xs[4 * q] + arow[rr][q].y * xs[4 * q + 1]) +
                                          (arow[rr][q].z * xs[4 * q + 2] + arow[rr][q].w * xs[4 * q + 3]);
                            float sum = part[0] + part[1];
                            sum += dpp_row<0xB1>(sum);   // quad_perm [1,0,3,2]: the partner lane
                            const float xr = (rr == j ? 1.f : 0.f) - sum;
                            const int pslot = 4 * (rr >> 3) + (rr & 3);
                            xs[pslot] = ((rr >> 2) & 1) == h ? xr : xs[pslot];
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        const float bj = sm.beta[b0 + j];
#pragma unroll
                        for (int q = 0; q < 8; ++q) {
                            const int row = b0 + 8 * (q >> 2) + 4 * h + (q & 3);
                            nm[row][b0 + j] = xs[q];
                            sm.tm[row][cc_pos<Cfg>(row, b0 + j)] = T::fromf(xs[q] * bj);
                        }
                    }
                } else {
                    const int blk = lane >> 4, j = lane & 15;
                    if (blk < NBLK) {
                        const int b0 = 16 * blk;
                        float x[16];   // column j of the block, rows 0..15
                        // A's rows, read two rows ahead of their use (the
                        // scheduling barriers keep that order: left alone, the
                        // compiler issues each row's reads just before it)
                        float4 arow[16][4];
                        auto read_row = [&](int rr) {
#pragma unroll
                            for (int m4 = 0; 4 * m4 < rr; ++m4)
                                arow[rr][m4] = *reinterpret_cast<const float4*>(&lm[b0 + rr][b0 + 4 * m4]);
                        };
                        read_row(1);
                        read_row(2);
#pragma unroll
                        for (int rr = 0; rr < 16; ++rr) {
                            if (rr + 2 < 16) read_row(rr + 2);
                            // one partial sum per group of four earlier rows, so
                            // that only the newest group waits on row rr - 1
                            float part[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int m4 = 0; 4 * m4 < rr; ++m4) {
                                const float av[4] = {arow[rr][m4].x, arow[rr][m4].y, arow[rr][m4].z, arow[rr][m4].w};
#pragma unroll
                                for (int i = 0; i < 4; ++i)
                                    if (4 * m4 + i < rr) part[m4] += av[i] * x[4 * m4 + i];
                            }
                            x[rr] = (rr == j ? 1.f : 0.f) - ((part[0] + part[1]) + (part[2] + part[3]));
                            __builtin_amdgcn_sched_barrier(0);
                        }
                        const float bj = sm.beta[b0 + j];
#pragma unroll
                        for (int m = 0; m < 16; ++m) {
                            nm[b0 + m][b0 + j] = x[m];
                            sm.tm[b0 + m][cc_pos<Cfg>(b0 + m, b0 + j)] = T::fromf(x[m] * bj);
                        }
                    }
                }
            }
            // P on the other waves (on every wave when there are fewer than 4)
            constexpr int P0 = SOLVE2 ? 2 : NW >= 4 ? 1 : 0, PW = NW - P0;
            if (wave >= P0) {
                int idx = 0;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                    for (int sb = 0; sb <= tb; ++sb, ++idx) {
                        if (idx % PW != wave - P0) continue;
                        f32x4_t ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int kk = 0; kk < D / MK; ++kk)
                            ap = T::mma(row_frag<Cfg, DM>(&sm.k[0][0], D, 16 * sb, kk * MK, lane),
                                        row_frag<Cfg, DM>(&sm.q[0][0], D, 16 * tb, kk * MK, lane), ap);
                        const int t = 16 * tb + r, s0 = 16 * sb + 4 * g;
                        float xp[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) xp[i] = s0 + i <= t ? ap[i] : 0.f;
                        store_run<BF16, 4>(&sm.pm[t][cc_pos<Cfg>(t, s0)], xp);
                    }
            }
            form_xt();
        }
        __syncthreads();

        // S^T Q^T of the output, formed by the waves other than wave 0 while
        // wave 0 runs the longest off-diagonal chain (it involves neither T
        // nor this chunk's update; V - K S there as well measured slower: the
        // chain is short enough that the two products outlast it)
        f32x4_t oq[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) oq[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        // ---- the blocks below the diagonal, one block column per wave (the
        // blocks of column j need only N_jj, the diagonal blocks and the
        // column's own earlier blocks, so no workgroup barrier between them):
        // N_ij = -N_ii sum_{j <= m < i} A_im N_mj, and T_ij = N_ij beta_j.
        // The column's blocks stay in registers: a product's result (lane
        // slot i holding row 4 g + i) is the next product's B operand with
        // the k index 4 g + i at step i, the A operand read from LDS to match
#pragma unroll
        for (int jb = 0; jb < NBLK - 1; ++jb) {
            if (jb % NW != wave) continue;   // uniform: compile-time block indices below
            const int bj = 16 * jb;
            const float betj = sm.beta[bj + r];
            if constexpr (BF16) {
                // bf16 inputs: the products on 16x16x16 bf16 matrix cores (one
                // instruction per block product, against four fp32 ones),
                // whose B operand is a result's accumulator layout as it
                // stands (k = 4 g + i in slot i); A, the diagonal blocks of N
                // and the column's blocks rounded to bf16 as operands, sums in
                // fp32 (T itself is stored in bf16)
                auto pk4 = [](float a, float b, float c, float d) {
                    return __builtin_bit_cast(bw_i16x4, make_uint2(pack_bf16(a, b), pack_bf16(c, d)));
                };
                auto row4 = [&](const float* p) {
                    const float4 v = *reinterpret_cast<const float4*>(p);
                    return pk4(v.x, v.y, v.z, v.w);
                };
                const bw_i16x4 njj = pk4(nm[bj + 4 * g][bj + r], nm[bj + 4 * g + 1][bj + r],
                                         nm[bj + 4 * g + 2][bj + r], nm[bj + 4 * g + 3][bj + r]);
                bw_i16x4 nbp[NBLK];   // N_mj, m > jb, as B operands
#pragma unroll
                for (int ib = jb + 1; ib < NBLK; ++ib) {
                    const int bi = 16 * ib;
                    f32x4_t xm[NBLK];
                    xm[jb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(row4(&lm[bi + r][bj + 4 * g]), njj,
                                                                      f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                    for (int m = jb + 1; m < ib; ++m)
                        xm[m] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(row4(&lm[bi + r][16 * m + 4 * g]), nbp[m],
                                                                         f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    f32x4_t x = xm[jb];
#pragma unroll
                    for (int m = jb + 1; m < ib; ++m) x += xm[m];
                    const f32x4_t y = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
                        row4(&nm[bi + r][bi + 4 * g]), pk4(x[0], x[1], x[2], x[3]), f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    nbp[ib] = pk4(-y[0], -y[1], -y[2], -y[3]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = bi + 4 * g + i;
                        sm.tm[row][cc_pos<Cfg>(row, bj + r)] = T::fromf(-y[i] * betj);
                    }
                }
            } else {
                f32x4_t nb[NBLK];   // N_mj, m > jb: slot i holds row 16 m + 4 g + i, column bj + r
#pragma unroll
                for (int ib = jb + 1; ib < NBLK; ++ib) {
                    const int bi = 16 * ib;
                    // one accumulator per term, so the products do not wait on each other
                    f32x4_t xm[NBLK];
                    xm[jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xm[jb] = F::mma(lm[bi + r][bj + 4 * g + i], nm[bj + 4 * g + i][bj + r], xm[jb]);
#pragma unroll
                    for (int m = jb + 1; m < ib; ++m) {
                        xm[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int i = 0; i < 4; ++i) xm[m] = F::mma(lm[bi + r][16 * m + 4 * g + i], nb[m][i], xm[m]);
                    }
                    f32x4_t x = xm[jb];
#pragma unroll
                    for (int m = jb + 1; m < ib; ++m) x += xm[m];
                    f32x4_t y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int i = 0; i < 4; ++i) y = F::mma(nm[bi + r][bi + 4 * g + i], x[i], y);
                    nb[ib] = -y;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = bi + 4 * g + i;
                        sm.tm[row][cc_pos<Cfg>(row, bj + r)] = T::fromf(-y[i] * betj);
                    }
                }
            }
        }
        // the next chunk's loads: issued here, where the waves without a block
        // column would otherwise wait for the off-diagonal chain (the
        // registers were emptied into this chunk's tiles)
        if (c + 1 < nchunks) load(c + 1);
        if (HELP && wave == HW) {
            // its own S^T Q^T and wave 0's, over the same Q fragments; wave
            // 0's handed back through LDS (read after the next barrier)
            if constexpr (HELP) {
                Frag s0[D / 32];
#pragma unroll
                for (int k2 = 0; k2 < D / 32; ++k2) s0[k2] = __builtin_bit_cast(Frag, sm.sa0[k2][lane]);
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    f32x4_t o0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int k2 = 0; k2 < D / 32; ++k2) {
                        const Frag qf = x_frag(&sm.q[0][0], tb, k2);
                        oq[tb] = T::mma(sa[k2], qf, oq[tb]);
                        o0 = T::mma(s0[k2], qf, o0);
                    }
                    sm.oq0[tb][lane] = o0;
                }
            }
        } else if (wave != 0) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) oq[tb] = state_times(&sm.q[0][0], tb, oq[tb]);
        }
        __syncthreads();

        // ---- U' = T (V - K S) for this wave's value columns: V - K S as the
        // B operand (k-slots tokens 32 k2 + 4 g + i and 32 k2 + 16 + 4 g + i,
        // T read to match); lane slot i of ut[sb] holds token 16 sb + 4 g + i
        f32x4_t ut[TB];
        if constexpr (BF16) {
            Frag xf[C / 32];
#pragma unroll
            for (int k2 = 0; k2 < C / 32; ++k2) {
                const float x8[8] = {xt[2 * k2][0], xt[2 * k2][1], xt[2 * k2][2], xt[2 * k2][3],
                                     xt[2 * k2 + 1][0], xt[2 * k2 + 1][1], xt[2 * k2 + 1][2],
                                     xt[2 * k2 + 1][3]};
                xf[k2] = T::from8(x8);
            }
#pragma unroll
            for (int sb = 0; sb < TB; ++sb) {
                const int s = 16 * sb + r;
                ut[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k2 = 0; k2 <= sb / 2; ++k2)
                    ut[sb] = T::mma(T::load2x4(&sm.tm[s][cc_pos<Cfg>(s, 32 * k2 + 4 * g)],
                                               &sm.tm[s][cc_pos<Cfg>(s, 32 * k2 + 16 + 4 * g)]),
                                    xf[k2], ut[sb]);
            }
        } else {
#pragma unroll
            for (int sb = 0; sb < TB; ++sb) {
                const int s = 16 * sb + r;
                ut[sb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int xb = 0; xb <= sb; ++xb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        ut[sb] = T::mma(sm.tm[s][cc_pos<Cfg>(s, 16 * xb + 4 * g + i)], xt[xb][i], ut[sb]);
            }
        }

        // ---- O^T = S^T Q^T + U'^T P^T, then S += K^T U', with U' as the
        // operand in the same token order (P and K read to match)
        Frag uf[BF16 ? C / 32 : 1];
        if constexpr (BF16) {
#pragma unroll
            for (int k2 = 0; k2 < C / 32; ++k2) {
                const float x8[8] = {ut[2 * k2][0], ut[2 * k2][1], ut[2 * k2][2], ut[2 * k2][3],
                                     ut[2 * k2 + 1][0], ut[2 * k2 + 1][1], ut[2 * k2 + 1][2],
                                     ut[2 * k2 + 1][3]};
                uf[k2] = T::from8(x8);
            }
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            f32x4_t acc;
            if constexpr (HELP) acc = wave != 0 ? oq[tb] : sm.oq0[tb][lane];
            else acc = wave != 0 ? oq[tb] : state_times(&sm.q[0][0], tb, oq[tb]);
            const int t = 16 * tb + r;
            if constexpr (BF16) {
#pragma unroll
                for (int k2 = 0; k2 <= tb / 2; ++k2)
                    acc = T::mma(uf[k2],
                                 T::load2x4(&sm.pm[t][cc_pos<Cfg>(t, 32 * k2 + 4 * g)],
                                            &sm.pm[t][cc_pos<Cfg>(t, 32 * k2 + 16 + 4 * g)]),
                                 acc);
            } else {
#pragma unroll
                for (int sb = 0; sb <= tb; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        acc = T::mma(ut[sb][i], sm.pm[t][cc_pos<Cfg>(t, 16 * sb + 4 * g + i)], acc);
            }
            const uint32_t off = ((uint32_t)(t0 + t) * D + n0 + 4 * g) * ES;
            float xo[4] = {acc[0], acc[1], acc[2], acc[3]};
            buf_store_run4<BF16>(ro, off, xo);
        }
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
            if constexpr (BF16) {
                // K^T: state rows 16 mb + r, k-slots tokens 32 k2 + 4 g + i
                // and 32 k2 + 16 + 4 g + i (two transposing reads)
#pragma unroll
                for (int k2 = 0; k2 < C / 32; ++k2) {
                    const int rowa = 32 * k2 + 4 * g + (r >> 2), rowb = rowa + 16;
                    const int col = 16 * mb + 4 * (r & 3);
                    const bw_i16x4 ka = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) bw_i16x4*)(&sm.k[rowa][bw_pos<Cfg, DM>(rowa, col)]));
                    const bw_i16x4 kb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) bw_i16x4*)(&sm.k[rowb][bw_pos<Cfg, DM>(rowb, col)]));
                    const uint2 ua = __builtin_bit_cast(uint2, ka), ub = __builtin_bit_cast(uint2, kb);
                    accS[mb] = T::mma(__builtin_bit_cast(Frag, make_uint4(ua.x, ua.y, ub.x, ub.y)), uf[k2],
                                      accS[mb]);
                }
            } else {
#pragma unroll
                for (int sb = 0; sb < TB; ++sb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * sb + 4 * g + i;
                        accS[mb] = T::mma(sm.k[row][bw_pos<Cfg, DM>(row, 16 * mb + r)], ut[sb][i], accS[mb]);
                    }
            }
        }
        __syncthreads();
    }

    if (p.S_final) {
        float* Sf = p.S_final + (size_t)bh * D * D;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Sf[(size_t)(16 * mb + 4 * g + i) * D + n0 + r] = accS[mb][i];
    }
}

// Decode: one step of the delta rule per (b,h).
template <int D>
struct DeltaDecodeShape {
    static constexpr int NT = D >= 128 ? 512 : 256;
};

template <int D, bool BF16>
__global__ __launch_bounds__((DeltaDecodeShape<D>::NT)) void delta_decode_kernel(const DeltaParams p) {
    using T = Elem<BF16>;
    using E = typename T::E;
    constexpr int NT = DeltaDecodeShape<D>::NT;
    constexpr int CQ = D / 4;                 // column quads per row
    constexpr int RPP = NT / CQ;              // rows per pass
    constexpr int NPASS = (D + RPP - 1) / RPP;
    static_assert(NT % CQ == 0, "column quads must divide the workgroup");

    __shared__ float sq[D], sk[D], sv[D], su[D], sw[D];
    __shared__ float4 redu[RPP][CQ], redw[RPP][CQ];
    __shared__ float sqk;

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const E* q = reinterpret_cast<const E*>(p.q) + (size_t)bh * D;
    const E* k = reinterpret_cast<const E*>(p.k) + (size_t)bh * D;
    const E* v = reinterpret_cast<const E*>(p.v) + (size_t)bh * D;
    f32x4_t* S = reinterpret_cast<f32x4_t*>(p.S + (size_t)bh * D * D);
    const float beta = p.beta[bh];

    const int cq = tid % CQ, rr = tid / CQ;
    f32x4_t sreg[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPP + rr;
        if (row < D) sreg[ps] = __builtin_nontemporal_load(&S[(size_t)row * CQ + cq]);
    }
    if (tid < D) {
        sq[tid] = T::tof(q[tid]);
        sk[tid] = T::tof(k[tid]);
        sv[tid] = T::tof(v[tid]);
    }
    __syncthreads();

    // u = S^T k and w = S^T q: this thread's rows, then the row groups
    float4 pu = make_float4(0.f, 0.f, 0.f, 0.f), pw = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPP + rr;
        if (row < D) {
            const float kk = sk[row], qq = sq[row];
            const f32x4_t s = sreg[ps];
            pu.x += kk * s[0]; pu.y += kk * s[1]; pu.z += kk * s[2]; pu.w += kk * s[3];
            pw.x += qq * s[0]; pw.y += qq * s[1]; pw.z += qq * s[2]; pw.w += qq * s[3];
        }
    }
    redu[rr][cq] = pu;
    redw[rr][cq] = pw;
    if (tid == 0) {
        float a = 0.f;
        for (int i = 0; i < D; ++i) a += sq[i] * sk[i];
        sqk = a;
    }
    __syncthreads();
    if (tid < D) {
        const int c4 = tid >> 2, e = tid & 3;
        float u = 0.f, w = 0.f;
        for (int j = 0; j < RPP; ++j) {
            const float4 a = redu[j][c4], b = redw[j][c4];
            u += e == 0 ? a.x : e == 1 ? a.y : e == 2 ? a.z : a.w;
            w += e == 0 ? b.x : e == 1 ? b.y : e == 2 ? b.z : b.w;
        }
        su[tid] = u;
        sw[tid] = w;
    }
    __syncthreads();

    // S += beta k (v - u)^T, o = w + beta (q . k) (v - u)
    const float4 vv = *reinterpret_cast<const float4*>(&sv[4 * cq]);
    const float4 uu = *reinterpret_cast<const float4*>(&su[4 * cq]);
    const float4 dlt = make_float4(beta * (vv.x - uu.x), beta * (vv.y - uu.y),
                                   beta * (vv.z - uu.z), beta * (vv.w - uu.w));
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPP + rr;
        if (row < D) {
            const float kk = sk[row];
            f32x4_t s = sreg[ps];
            s[0] += kk * dlt.x;
            s[1] += kk * dlt.y;
            s[2] += kk * dlt.z;
            s[3] += kk * dlt.w;
            __builtin_nontemporal_store(s, &S[(size_t)row * CQ + cq]);
        }
    }
    if (tid < D) {
        const float o = sw[tid] + beta * sqk * (sv[tid] - su[tid]);
        reinterpret_cast<E*>(p.out)[(size_t)bh * D + tid] = T::fromf(o);
    }
}

// Chunk length of the delta prefill: 64 tokens, 32 for fp32 at d = 128
// (LDS).
constexpr int delta_chunk(int d, bool bf16) { return (!bf16 && d >= 128) ? 32 : 64; }

template <int D, bool BF>
hipError_t launch_delta_dt(const DeltaParams& p, bool decode, hipStream_t s) {
    if (decode) {
        LA_LAUNCH((delta_decode_kernel<D, BF>), dim3(p.BH), dim3(DeltaDecodeShape<D>::NT), s, p);
    } else {
        using Cfg = DeltaCfg<D, delta_chunk(D, BF), BF>;
        LA_LAUNCH((delta_chunk_kernel<Cfg>), dim3(p.BH), dim3(Cfg::NT), s, p);
    }
    return hipGetLastError();
}

#define LA_DEFINE_DELTA_LAUNCHER(NAME, D, BF) \
    hipError_t NAME(const DeltaParams& p, bool decode, hipStream_t s) { return launch_delta_dt<D, BF>(p, decode, s); }

}  // namespace la
