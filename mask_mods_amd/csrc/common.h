// common.h -- device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type tags for the two 16-bit MFMA input types.
struct BF16 {
    typedef bf16x8 vec8;
    typedef bf16x4 vec4;
};
struct F16 {
    typedef f16x8 vec8;
    typedef f16x4 vec4;
};

// 32x32x16 MFMA, fp32 accumulate. Operand lane layout (wave64):
//   A[m][k]: lane l holds m = l % 32, k = 8*(l / 32) + 0..7
//   B[k][n]: lane l holds n = l % 32, k = 8*(l / 32) + 0..7
//   C[m][n]: lane l, element e holds n = l % 32, m = 8*(e / 4) + 4*(l / 32) + e % 4
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x16(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// 16 bytes <-> 8-element vectors
template <typename V>
__device__ __forceinline__ V as_vec(u32x4 x) { return __builtin_bit_cast(V, x); }

// fp32 -> 16-bit, round to nearest even
__device__ __forceinline__ bf16x8 cvt8(f32x8 x, BF16) { return __builtin_convertvector(x, bf16x8); }
__device__ __forceinline__ f16x8 cvt8(f32x8 x, F16) { return __builtin_convertvector(x, f16x8); }
__device__ __forceinline__ bf16x4 cvt4(f32x4 x, BF16) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ f16x4 cvt4(f32x4 x, F16) { return __builtin_convertvector(x, f16x4); }

// 16-bit -> fp32 (exact)
__device__ __forceinline__ f32x8 widen8(u32x4 x, BF16) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x8, x), f32x8);
}
__device__ __forceinline__ f32x8 widen8(u32x4 x, F16) {
    return __builtin_convertvector(__builtin_bit_cast(f16x8, x), f32x8);
}
__device__ __forceinline__ float widen1(uint16_t x, BF16) {
    return __uint_as_float(((uint32_t)x) << 16);
}
__device__ __forceinline__ float widen1(uint16_t x, F16) {
    return (float)__builtin_bit_cast(_Float16, x);
}

__device__ __forceinline__ uint16_t narrow1(float x, BF16) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ uint16_t narrow1(float x, F16) { return __builtin_bit_cast(uint16_t, (_Float16)x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MurmurHash3 32-bit finalizer (Austin Appleby, public domain).
__host__ __device__ __forceinline__ uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

// Blocks are handed to the 8 XCDs round-robin (block p runs on XCD p % 8). Remap so
// each XCD receives a contiguous range of logical blocks: neighbouring logical blocks
// (same head, adjacent query tiles) then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int p, int n) {
    const int nx = 8;
    const int q = n / nx, r = n % nx;
    const int x = p % nx, s = p / nx;
    return x * q + (x < r ? x : r) + s;
}

// Work item of workgroup p of n = n_tiles * pairs (pairs = (batch, head) rows): its tile
// index and its pair. Plain: the XCD remap above, tiles fastest, so all the tiles of a
// pair share one XCD's L2. Causal (heavy = true: tile t carries about t + 1 units of
// work): tile-major over the whole grid, heaviest tiles first, so that the dispatcher
// starts every pair's longest tile before any shorter one and the short tiles fill in
// at the end (longest-first list scheduling); workgroups go to the XCDs round-robin by
// id, so with pairs a multiple of 8 a pair's tiles still share an XCD.
__device__ __forceinline__ void work_item(int p, int n, int n_tiles, bool heavy_last, int &tile, int &pair) {
    if (heavy_last) {
        const int pairs = n / n_tiles;
        tile = n_tiles - 1 - p / pairs;
        pair = p % pairs;
    } else {
        const int L = xcd_remap(p, n);
        tile = L % n_tiles;
        pair = L / n_tiles;
    }
}

// On a non-decreasing int32 array of n entries: the first index whose value is >= v
// (lower) or > v (upper); n if none.
__device__ __forceinline__ int doc_lower(const int32_t *a, int n, int v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < v) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}
__device__ __forceinline__ int doc_upper(const int32_t *a, int n, int v) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] <= v) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

}  // namespace mm
