// la_device.h -- device-side helpers for the gfx950 kernels: bf16 packing,
// matrix-core (MFMA) wrappers and fragment loaders.
//
// Matrix-core conventions used throughout (16x16 output tiles, wave64):
//   lane = 16*g + r  with  r = lane & 15, g = lane >> 4 (0..3)
//   A operand (16 x K):  lane holds row m = r, k-slots j of k-group g
//   B operand (K x 16):  lane holds column n = r, k-slots j of k-group g
//   C/D (16 x 16 fp32):  lane holds D[4g + i][r], i = 0..3
// bf16 (v_mfma_f32_16x16x32_bf16): K = 32, 8 k-slots per lane, and the
// k index of (g, j) is 8g + j for A and B alike.  fp32
// (v_mfma_f32_16x16x4_f32): K = 4, one k-slot per lane, k = g.  Only the
// pairing "same (g, j) in A and B" matters for a contraction, so operands
// may permute k as long as both sides use the same permutation.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;

// ---------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16hi(uint32_t p) { return __uint_as_float(p & 0xffff0000u); }
__device__ __forceinline__ float bf16f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats -> two bf16 (round to nearest even) packed low/high.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    f32x2_t v = {lo, hi};
    bf16x2_t h = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}
__device__ __forceinline__ uint16_t to_bf16(float x) {
    return (uint16_t)(pack_bf16(x, 0.0f) & 0xffffu);
}

// ---------------------------------------------------------------- element traits
// E is the element type of LDS tiles and matrix-core operands: uint16_t
// (bf16 bits) for bf16 inputs, float for fp32 inputs.
template <bool BF16> struct Elem;
template <> struct Elem<true> {
    using E = uint16_t;
    using Pair = uint32_t;            // two adjacent bf16 of a row
    using Frag = bf16x8_t;            // one matrix-core operand per lane
    static constexpr int KPL = 8;     // k-slots per lane
    static constexpr int MK = 32;     // K of one instruction
    __device__ static float lo(Pair p) { return bf16lo(p); }
    __device__ static float hi(Pair p) { return bf16hi(p); }
    __device__ static Pair pack(float a, float b) { return pack_bf16(a, b); }
    __device__ static float tof(E e) { return bf16f(e); }
    __device__ static E fromf(float x) { return to_bf16(x); }
    __device__ static Pair zero() { return 0u; }
    __device__ static f32x4_t mma(Frag a, Frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // KPL contiguous elements starting at p (16-byte aligned)
    __device__ static Frag load(const E* p) {
        return __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(p));
    }
    // two runs of 4 contiguous elements (8-byte aligned each)
    __device__ static Frag load2x4(const E* p0, const E* p1) {
        uint2 a = *reinterpret_cast<const uint2*>(p0);
        uint2 b = *reinterpret_cast<const uint2*>(p1);
        uint4 u = {a.x, a.y, b.x, b.y};
        return __builtin_bit_cast(Frag, u);
    }
    // 8 fp32 -> fragment (RNE)
    __device__ static Frag from8(const float* x) {
        uint4 u = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]),
                   pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
        return __builtin_bit_cast(Frag, u);
    }
};
template <> struct Elem<false> {
    using E = float;
    using Pair = float2;
    using Frag = float;
    static constexpr int KPL = 1;
    static constexpr int MK = 4;
    __device__ static float lo(Pair p) { return p.x; }
    __device__ static float hi(Pair p) { return p.y; }
    __device__ static Pair pack(float a, float b) { return make_float2(a, b); }
    __device__ static float tof(E e) { return e; }
    __device__ static E fromf(float x) { return x; }
    __device__ static Pair zero() { return make_float2(0.f, 0.f); }
    __device__ static f32x4_t mma(Frag a, Frag b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
    }
    __device__ static Frag load(const E* p) { return *p; }
};

// Store N consecutive elements held as N/2 pairs (row segment of an LDS
// tile) with the widest aligned vector stores available.
template <bool BF16, int N>
__device__ __forceinline__ void store_run(typename Elem<BF16>::E* dst, const float* x) {
    if constexpr (BF16) {
        static_assert(N % 2 == 0, "bf16 runs are stored as pairs");
        uint32_t w[N / 2];
#pragma unroll
        for (int j = 0; j < N / 2; ++j) w[j] = pack_bf16(x[2 * j], x[2 * j + 1]);
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int j = 0; j < N / 8; ++j)
                reinterpret_cast<uint4*>(dst)[j] = make_uint4(w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]);
        } else if constexpr (N % 4 == 0) {
#pragma unroll
            for (int j = 0; j < N / 4; ++j)
                reinterpret_cast<uint2*>(dst)[j] = make_uint2(w[2 * j], w[2 * j + 1]);
        } else {
#pragma unroll
            for (int j = 0; j < N / 2; ++j) reinterpret_cast<uint32_t*>(dst)[j] = w[j];
        }
    } else {
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int j = 0; j < N / 4; ++j)
                reinterpret_cast<float4*>(dst)[j] = make_float4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3]);
        } else if constexpr (N % 2 == 0) {
#pragma unroll
            for (int j = 0; j < N / 2; ++j)
                reinterpret_cast<float2*>(dst)[j] = make_float2(x[2 * j], x[2 * j + 1]);
        } else {
#pragma unroll
            for (int j = 0; j < N; ++j) dst[j] = x[j];
        }
    }
}

// A run of adjacent channels of one token as raw 32-bit words.
template <int N>
struct Words {
    uint32_t w[N];
};
// Channel c of a run as a float (bf16 runs hold two channels per word).
template <bool BF16, int N>
__device__ __forceinline__ float run_elem(const Words<N>& x, int c) {
    if constexpr (BF16) return (c & 1) ? bf16hi(x.w[c >> 1]) : bf16lo(x.w[c >> 1]);
    else return __uint_as_float(x.w[c]);
}
// N floats as a run of the tile element type.
template <bool BF16, int N>
__device__ __forceinline__ Words<(BF16 ? N / 2 : N)> pack_run(const float* x) {
    Words<(BF16 ? N / 2 : N)> o;
    if constexpr (BF16) {
#pragma unroll
        for (int i = 0; i < N / 2; ++i) o.w[i] = pack_bf16(x[2 * i], x[2 * i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) o.w[i] = __float_as_uint(x[i]);
    }
    return o;
}
template <int N>
__device__ __forceinline__ void lds_store_words(void* p, const Words<N>& x) {
    if constexpr (N == 1) *reinterpret_cast<uint32_t*>(p) = x.w[0];
    else if constexpr (N == 2) *reinterpret_cast<uint2*>(p) = make_uint2(x.w[0], x.w[1]);
    else *reinterpret_cast<uint4*>(p) = make_uint4(x.w[0], x.w[1], x.w[2], x.w[3]);
}
// Value of x in lane src of the wave (an LDS-crossbar permute).
__device__ __forceinline__ float lane_read(float x, int src) {
    return __int_as_float(__builtin_amdgcn_ds_bpermute(src << 2, __float_as_int(x)));
}
// x of the lane that the DPP control CTRL selects within the lane's 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp_sel(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum of x over each aligned group of N adjacent lanes (N = 1, 2, 4, 8 or
// 16), received by every lane of the group, in DPP moves inside a 16-lane
// row: rotations by 8 and 4 (N = 16) or the half-row mirror (N = 8) gather
// the lanes that are equal modulo 4, then the quad permutations [2,3,0,1]
// and [1,0,3,2] add the four residues.
template <int N>
__device__ __forceinline__ float lane_group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "groups of 1 to 16 lanes");
    if constexpr (N == 16) {
        x += dpp_sel<0x128>(x);    // row_ror:8
        x += dpp_sel<0x124>(x);    // row_ror:4
    }
    if constexpr (N == 8) x += dpp_sel<0x141>(x);    // row_half_mirror
    if constexpr (N >= 4) x += dpp_sel<0x4E>(x);     // quad_perm [2,3,0,1]
    if constexpr (N >= 2) x += dpp_sel<0xB1>(x);     // quad_perm [1,0,3,2]
    return x;
}
// Buffer descriptor over [base, base + bytes); reads past the end return 0
// and writes past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// AUX is the cache policy of the load: 0 by default, LOAD_NT (the nt,
// non-temporal bit) for streams read once.
constexpr int LOAD_NT = 2;
template <int N, int AUX = 0>
__device__ __forceinline__ Words<N> buf_load_words(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (N == 1) {
        return Words<1>{{__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX)}};
    } else if constexpr (N == 2) {
        return __builtin_bit_cast(Words<2>, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX));
    } else {
        static_assert(N == 4, "runs are 4, 8 or 16 bytes");
        return __builtin_bit_cast(Words<4>, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
    }
}


// A run of 4 channels of one token (fp32 values) written to global memory as
// the element type through a buffer descriptor.
template <bool BF16>
__device__ __forceinline__ void buf_store_run4(__amdgpu_buffer_rsrc_t r, uint32_t off, const float* x) {
    if constexpr (BF16) {
        const u32x2_t w = {pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3])};
        __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, 0);
    } else {
        const f32x4_t v = {x[0], x[1], x[2], x[3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 0);
    }
}

// phi = elu + 1 (x + 1 for x > 0, exp(x) otherwise) or identity.
__device__ __forceinline__ float feature(float x, int elu1) {
    return elu1 ? (x > 0.0f ? x + 1.0f : __expf(x)) : x;
}
// elu + 1 without a branch (both sides evaluated, then selected).
__device__ __forceinline__ float elu1f(float x) {
    const float e = __expf(fminf(x, 0.0f));
    return x > 0.0f ? x + 1.0f : e;
}

}  // namespace la
