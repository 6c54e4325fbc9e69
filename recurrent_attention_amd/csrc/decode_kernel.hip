// decode_kernel.hip -- one recurrent step per (b,h): the recurrent face of
// the unified recurrence ("Module 22: Linear & Recurrent Attention",
// incremental decoding with a running state and the one-recurrence gate
// table; "causal linear attention as an RNN", O(1) state per step):
//
//   S <- A S + phi(k) v^T,  z <- A z + phi(k),  o = phi(q)^T S [/ phi(q).z]
//
// The step is a streaming read-modify-write of the fp32 state (64 KiB per
// pair at d = 128), so it is HBM-bound.  One workgroup per pair (512 threads
// at d = 128, where that streams best, else 256): each thread owns a quad of
// consecutive columns (16-byte non-temporal accesses, a whole 512-byte row
// per 32 threads) over DK / rows-per-pass rows, issues all its state loads
// before using them and keeps the updated rows in registers; the partial
// outputs of the row groups are reduced through LDS, and the updated rows
// are stored after that barrier, at lowered wave priority.
#include "la_device.h"
#include "la_internal.h"

namespace la {

template <int DK, int DV>
struct DecodeShape {
    static constexpr int NT = DK * DV >= 128 * 128 ? 512 : 256;   // threads
};

// four waves per SIMD (up to 128 registers; two 512-thread workgroups,
// 128 KiB of state reads, in flight per CU) stream as fast as eight, which
// would cap the kernel at 64 registers and spill the held rows to scratch
template <int DK, int DV, bool BF16, int GATE>
__global__ __launch_bounds__((DecodeShape<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(4, 4)))
void decode_kernel(const DecodeParams p) {
    using T = Elem<BF16>;
    using E = typename T::E;
    constexpr int NT = DecodeShape<DK, DV>::NT;
    constexpr int CQ = DV / 4;               // column quads per row
    constexpr int RPP = NT / CQ;             // rows per pass
    constexpr int NPASS = (DK + RPP - 1) / RPP;
    static_assert(NT % CQ == 0, "column quads must divide the workgroup");

    __shared__ float sq[DK], sk[DK], sa[DK], sqz[DK];
    __shared__ float sv[DV];
    __shared__ float sred[RPP][DV];

    const int tid = threadIdx.x;
    const int bh = blockIdx.x;
    const int h = bh % p.H;
    const int elu1 = p.phi_elu1;
    const bool norm = p.normalize != 0;

    const E* q = reinterpret_cast<const E*>(p.q) + (size_t)bh * DK;
    const E* k = reinterpret_cast<const E*>(p.k) + (size_t)bh * DK;
    const E* v = reinterpret_cast<const E*>(p.v) + (size_t)bh * DV;
    f32x4_t* S = reinterpret_cast<f32x4_t*>(p.S + (size_t)bh * DK * DV);

    const int cq = tid % CQ, rr = tid / CQ;
    // the waves issue their loads at raised priority and drop it before the
    // stores: with two workgroups per CU, the instruction arbiter then serves
    // one workgroup's state loads ahead of the other's trailing stores
    // (187.5 -> 176.5 us per step at 256 x 32 pairs, d = 128)
    __builtin_amdgcn_s_setprio(2);
    // issue the state loads first: they are the whole cost of the step
    f32x4_t sreg[NPASS];
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPP + rr;
        if (row < DK) sreg[ps] = __builtin_nontemporal_load(&S[(size_t)row * CQ + cq]);
    }

    if (tid < DK) {
        sq[tid] = feature(T::tof(q[tid]), elu1);
        sk[tid] = feature(T::tof(k[tid]), elu1);
        float a = 1.0f;
        if constexpr (GATE == LA_GATE_GAMMA) a = p.gamma[h];
        if constexpr (GATE == LA_GATE_DIAG) a = __expf(p.log_alpha[(size_t)bh * DK + tid]);
        if constexpr (GATE == LA_GATE_SCALAR) a = __expf(p.log_alpha[bh]);
        sa[tid] = a;
    }
    if (tid < DV) sv[tid] = T::tof(v[tid]);
    __syncthreads();

    const float4 vv = *reinterpret_cast<const float4*>(&sv[4 * cq]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPP + rr;
        if (row < DK) {
            const float a = sa[row], kk = sk[row], qq = sq[row];
            f32x4_t s = sreg[ps];
            s[0] = a * s[0] + kk * vv.x;
            s[1] = a * s[1] + kk * vv.y;
            s[2] = a * s[2] + kk * vv.z;
            s[3] = a * s[3] + kk * vv.w;
            sreg[ps] = s;
            acc.x += qq * s[0];
            acc.y += qq * s[1];
            acc.z += qq * s[2];
            acc.w += qq * s[3];
        }
    }
    *reinterpret_cast<float4*>(&sred[rr][4 * cq]) = acc;
    if (norm && tid < DK) {
        float* z = p.z + (size_t)bh * DK;
        const float zn = sa[tid] * z[tid] + sk[tid];
        z[tid] = zn;
        sqz[tid] = sq[tid] * zn;
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);

#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
        const int row = ps * RPP + rr;
        if (row < DK) __builtin_nontemporal_store(sreg[ps], &S[(size_t)row * CQ + cq]);
    }
    if (tid < DV) {
        float o = 0.f;
#pragma unroll
        for (int j = 0; j < RPP; ++j) o += sred[j][tid];
        if (norm) {
            float den = 0.f;
            for (int i = 0; i < DK; ++i) den += sqz[i];
            o /= den;
        }
        reinterpret_cast<E*>(p.out)[(size_t)bh * DV + tid] = T::fromf(o);
    }
}

template <int DK, int DV, bool BF>
static hipError_t launch_decode_dt(const DecodeParams& p, int gate, hipStream_t s) {
    const dim3 grid(p.BH), block(DecodeShape<DK, DV>::NT);
    if (gate == LA_GATE_NONE) LA_LAUNCH((decode_kernel<DK, DV, BF, 0>), grid, block, s, p);
    else if (gate == LA_GATE_GAMMA) LA_LAUNCH((decode_kernel<DK, DV, BF, 1>), grid, block, s, p);
    else if (gate == LA_GATE_DIAG) LA_LAUNCH((decode_kernel<DK, DV, BF, 2>), grid, block, s, p);
    else if (gate == LA_GATE_SCALAR) LA_LAUNCH((decode_kernel<DK, DV, BF, 3>), grid, block, s, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_decode_kv(const DecodeParams& p, bool bf16, int gate, hipStream_t s) {
    return bf16 ? launch_decode_dt<DK, DV, true>(p, gate, s) : launch_decode_dt<DK, DV, false>(p, gate, s);
}

hipError_t launch_decode(const DecodeParams& p, int dk, int dv, bool bf16, int gate, hipStream_t s) {
    if (dk == dv) {
        switch (dk) {
            case 16: return launch_decode_kv<16, 16>(p, bf16, gate, s);
            case 32: return launch_decode_kv<32, 32>(p, bf16, gate, s);
            case 64: return launch_decode_kv<64, 64>(p, bf16, gate, s);
            case 128: return launch_decode_kv<128, 128>(p, bf16, gate, s);
            default: return hipErrorInvalidValue;
        }
    }
    if (dk == 64 && dv == 128) return launch_decode_kv<64, 128>(p, bf16, gate, s);
    if (dk == 128 && dv == 64) return launch_decode_kv<128, 64>(p, bf16, gate, s);
    return hipErrorInvalidValue;
}

}  // namespace la
