// fwd_tile.h -- the 16-bit forward kernels' K/V tile layout in LDS and P packing.
#pragma once

#include "fwd_common.h"

namespace mm {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack2(float a, float b, BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ uint32_t pack2(float a, float b, F16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, f16x2));
}

// Swizzled row-major tile of 16-bit elements, D per row.
template <int D>
struct Tile {
    static constexpr int ROWB = 2 * D;  // bytes per key row
    static constexpr int CH = D / 8;    // 16-byte chunks per row
    // The K reads hit 16 consecutive rows at one chunk, so swz must be a bijection on
    // the row index modulo 16 (D = 128; for D = 64, two rows share a 256-byte bank
    // window and swz of rows of equal parity must differ). The transposed V reads of a
    // half-wave hit 4 consecutive rows (4a .. 4a+3) x 4 consecutive chunks, so the high
    // bits of swz must differ across such rows: row 4a+b takes b in bits 2-3 (D = 128),
    // and rows 4a, 4a+2 differ in bit 2 (D = 64).
    __host__ __device__ static constexpr int swz(int r) {
        return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
    }
    __host__ __device__ static constexpr int off(int r, int c) { return r * ROWB + 16 * (c ^ swz(r)); }
};

// Stores a wave's 32 x D accumulator tile as 16-bit rows. acc[db][4*g4 + e] holds row
// l32 (lane & 31), dim 32*db + 8*g4 + 4*hi + e (hi = lane / 32), the S^T-side layout of
// the 32x32 MFMA; each value is multiplied by `mul` (the lane's own factor). The tile
// goes through `os`, the wave's own 32-row slice of free LDS in the K tile layout, and
// leaves as whole rows, 16 bytes per lane (a lane's own values are 8 bytes in each of 32
// rows per store instruction). Row rr goes to base + rr * ss, for rr < nrows.
template <typename TT, int D>
__device__ __forceinline__ void store_rows_via_lds(const f32x16 (&acc)[D / 32], float mul, unsigned char *os,
                                                   uint16_t *base, int64_t ss, int nrows, int lane) {
    typedef Tile<D> TL;
    const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const f32x4 x = {acc[db][4 * g4 + 0] * mul, acc[db][4 * g4 + 1] * mul,
                             acc[db][4 * g4 + 2] * mul, acc[db][4 * g4 + 3] * mul};
            *(typename TT::vec4 *)(os + TL::off(l32, 4 * db + g4) + 8 * hi) = cvt4(x, TT{});
        }
    }
    constexpr int RPS = 64 / TL::CH;  // rows per store instruction
#pragma unroll
    for (int i = 0; i < 32 / RPS; ++i) {
        const int rr = i * RPS + lane / TL::CH, c = lane % TL::CH;
        const u32x4 y = *(const u32x4 *)(os + TL::off(rr, c));
        if (rr < nrows) *(u32x4 *)(base + (int64_t)rr * ss + 8 * c) = y;
    }
}

}  // namespace mm
