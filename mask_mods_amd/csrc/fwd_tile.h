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

}  // namespace mm
