// tile_ops.h -- LDS tile addressing and matrix-core operand reads shared by
// the per-chunk kernels that keep their tiles row-major (one token or one
// state row per tile row, 16-byte units XOR-swizzled by the row).  A Cfg
// provides T (Elem<bf16?>), E, Frag, BF16, KPL and UE (elements per 16-byte
// unit).
#pragma once

#include "la_device.h"

namespace la {

typedef short bw_i16x4 __attribute__((ext_vector_type(4)));

// The unit XOR of row `row` in a tile with `mask`-wide swizzle.  For bf16
// rows of 16 units (256 bytes) it is row ^ (12 if the row is odd): gfx950
// serves a 16-byte read in four passes of 16 lanes (quads grouped by the
// parity of the quad index within each half-wave) and an 8-byte transposing
// read in two passes of 32 lanes, so the plain row index, which keeps the
// 16-row fragment reads and the 8-byte row reads free of bank conflicts,
// left every transposing read (4-row groups 8 rows apart) two-way
// conflicted; this one keeps all three conflict-free.  Other rows XOR the
// row's low bits.
template <class Cfg, int MASK>
__device__ __forceinline__ int bw_swz(int row) {
    if constexpr (Cfg::BF16 && MASK == 15) return (row ^ ((row & 1) * 12)) & 15;
    else return row & MASK;
}

// Position of column `col` in row `row` of a tile with `mask`-wide swizzle.
template <class Cfg, int MASK>
__device__ __forceinline__ int bw_pos(int row, int col) {
    const int u = col / Cfg::UE, e = col % Cfg::UE;
    return ((u ^ bw_swz<Cfg, MASK>(row)) * Cfg::UE) + e;
}

// Operand whose 16 rows/columns are tile columns c0..c0+15 and whose k-slots
// are tile rows k0 + (slots of this lane): the transposed read of a
// row-major tile.  bf16: two ds_read_b64_tr_b16 (4 rows each); fp32: one
// element.
template <class Cfg, int MASK>
__device__ __forceinline__ typename Cfg::Frag tr_frag(const typename Cfg::E* tile, int ld, int k0,
                                                      int c0, int lane) {
    using Frag = typename Cfg::Frag;
    const int g = lane >> 4;
    if constexpr (Cfg::BF16) {
        const int m = lane & 15;
        const int rowa = k0 + 8 * g + (m >> 2), rowb = rowa + 4;
        const int col = c0 + 4 * (m & 3);
        const auto* pa = tile + rowa * ld + bw_pos<Cfg, MASK>(rowa, col);
        const auto* pb = tile + rowb * ld + bw_pos<Cfg, MASK>(rowb, col);
        const bw_i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) bw_i16x4*)(pa));
        const bw_i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) bw_i16x4*)(pb));
        const uint2 ua = __builtin_bit_cast(uint2, a), ub = __builtin_bit_cast(uint2, b);
        return __builtin_bit_cast(Frag, make_uint4(ua.x, ua.y, ub.x, ub.y));
    } else {
        const int row = k0 + g, col = c0 + (lane & 15);
        return tile[row * ld + bw_pos<Cfg, MASK>(row, col)];
    }
}

// Operand whose 16 rows/columns are tile rows r0..r0+15 and whose k-slots
// are tile columns k0 + (slots of this lane): a direct read.
template <class Cfg, int MASK>
__device__ __forceinline__ typename Cfg::Frag row_frag(const typename Cfg::E* tile, int ld, int r0,
                                                       int k0, int lane) {
    const int row = r0 + (lane & 15);
    const int col = k0 + Cfg::KPL * (lane >> 4);
    return Cfg::T::load(tile + row * ld + bw_pos<Cfg, MASK>(row, col));
}

// The k-slots of an operand as floats.
template <class Cfg>
__device__ __forceinline__ void frag_floats(const typename Cfg::Frag& f, float* x) {
    if constexpr (Cfg::BF16) {
        const uint4 w = __builtin_bit_cast(uint4, f);
        const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = bf16lo(u[j]);
            x[2 * j + 1] = bf16hi(u[j]);
        }
    } else {
        x[0] = f;
    }
}

// x of the lane CTRL selects within the 16-lane row (a DPP row shift), 0
// where that lane lies outside the row.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Inclusive scan over the 16 lanes of a row (lanes r' <= r), or the suffix
// (lanes r' >= r) when SUFFIX: row_shr:n reads lane r - n, row_shl:n lane r + n.
template <bool SUFFIX>
__device__ __forceinline__ float row_scan16(float x) {
    constexpr int base = SUFFIX ? 0x100 : 0x110;
    x += dpp_row<base + 1>(x);
    x += dpp_row<base + 2>(x);
    x += dpp_row<base + 4>(x);
    x += dpp_row<base + 8>(x);
    return x;
}

}  // namespace la
