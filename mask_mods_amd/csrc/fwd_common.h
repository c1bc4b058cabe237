// fwd_common.h -- pieces shared by the forward kernels: the cross-half row max, the
// global -> LDS copy, and the barrier that closes each K/V tile.
#pragma once

#include "common.h"
#include "kernels.h"

namespace mm {

typedef float f32x2 __attribute__((ext_vector_type(2)));
#define MM_LDS __attribute__((address_space(3)))

// max of x over lanes l and l ^ 32 (the two halves holding one query row)
__device__ __forceinline__ float row_max2(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]), __builtin_bit_cast(float, (uint32_t)sw[1]));
}

// Global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4). The LDS destination
// is M0 + 16*lane. Written in asm so the compiler does not track the copy: it would
// otherwise wait for every copy in flight before reading any LDS buffer it cannot
// prove disjoint. The kernel orders copies and reads itself (kv_barrier). No output
// registers; the kernels leave nothing of their own in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // m0 is written on purpose (see above)
__device__ __forceinline__ void dma16_sbase(const void *gbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 ::"v"(voff), "s"(gbase), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma16_vaddr(const void *gaddr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 ::"v"(gaddr), "s"(lds) : "memory", "m0");
}
// 4 bytes per lane (64 lanes: 256 contiguous bytes), LDS destination M0 + 4*lane
__device__ __forceinline__ void dma4_vaddr(const void *gaddr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                 ::"v"(gaddr), "s"(lds) : "memory", "m0");
}
#pragma clang diagnostic pop
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(uintptr_t)(const MM_LDS void *)p;
}

// barrier for the K/V pipeline: waits until this wave has at most VMCNT copies in
// flight (older copies have landed: the vector-memory counter retires in order) and
// its LDS reads are done, then synchronises the workgroup.
template <int VMCNT>
__device__ __forceinline__ void kv_barrier() {
    static_assert(VMCNT >= 0 && VMCNT < 64, "vmcnt");
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt((VMCNT & 15) | ((VMCNT >> 4) << 14) | (7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

// Wave-wide search on a non-decreasing int32 array of n entries for both ends of a
// range: the first index whose value is >= vlo and the first whose value is > vhi (n if
// none). n, vlo and vhi are wave-uniform and every lane of the wave takes part. Each
// round probes up to 128 evenly spaced entries per search (two loads per lane, probe
// lane + 64 j at lo + (lane + 64 j) * step); the probes that lie before the answer form
// a prefix, counted with two ballots, and the answer lies between the last of them and
// the next probe. Up to 16384 entries take two rounds of dependent loads, the two
// searches sharing them so that all four loads of a lane are in flight together.
__device__ __forceinline__ void wave_search_range(const int32_t *a, int n, int vlo, int vhi, int lane,
                                                  int &out_lo, int &out_hi) {
    int lo1 = 0, hi1 = n, lo2 = 0, hi2 = n;
    while (lo1 < hi1 || lo2 < hi2) {
        const int st1 = (hi1 - lo1 + 127) >> 7, st2 = (hi2 - lo2 + 127) >> 7;
        int i1[2], i2[2], x1[2], x2[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            i1[j] = lo1 + (lane + 64 * j) * st1;
            i2[j] = lo2 + (lane + 64 * j) * st2;
            x1[j] = lo1 < hi1 ? a[min(i1[j], hi1 - 1)] : 0;
            x2[j] = lo2 < hi2 ? a[min(i2[j], hi2 - 1)] : 0;
        }
        int c1 = 0, c2 = 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            c1 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i1[j] < hi1 && x1[j] < vlo));
            c2 += __builtin_popcountll(__builtin_amdgcn_ballot_w64(i2[j] < hi2 && x2[j] <= vhi));
        }
        if (lo1 < hi1) {
            if (c1 == 0) hi1 = lo1;
            else {
                const int h = min(lo1 + c1 * st1, hi1);
                lo1 = lo1 + (c1 - 1) * st1 + 1;
                hi1 = h;
            }
        }
        if (lo2 < hi2) {
            if (c2 == 0) hi2 = lo2;
            else {
                const int h = min(lo2 + c2 * st2, hi2);
                lo2 = lo2 + (c2 - 1) * st2 + 1;
                hi2 = h;
            }
        }
    }
    out_lo = lo1;
    out_hi = lo2;
}

// The keys of one 64-key tile that share a row's document, for documents whose ids do
// not decrease along the keys: lane l holds t = the id of key k0 + l (clamped to the last
// key), and `mine` is the id of the lane's row. Sets [first, end) to the lane's
// document's keys as offsets in the tile. The loop visits each distinct document among
// the wave's rows once (rows are sorted too), starting from the first lane's.
__device__ __forceinline__ void tile_doc_range(int t, int mine, int &first, int &end) {
    first = 0;
    end = 0;
    int d = __builtin_amdgcn_readfirstlane(mine);
    for (;;) {
        const int a = __builtin_popcountll(__builtin_amdgcn_ballot_w64(t < d));
        const int e = __builtin_popcountll(__builtin_amdgcn_ballot_w64(t <= d));
        if (mine == d) {
            first = a;
            end = e;
        }
        const uint64_t later = __builtin_amdgcn_ballot_w64(mine > d);
        if (later == 0) break;
        d = __builtin_amdgcn_readlane(mine, __builtin_ctzll(later));
    }
}

// Walks the non-empty entries of one row of a block-mask table (one byte per key tile).
// The row is read 64 bytes at a time (one per lane) into a register window; a ballot of
// the nonzero bytes gives a wave-uniform bitmap, so every wave of a workgroup finds the
// same sequence of tiles without LDS, and a new window is loaded once per 64 tiles.
// Call next() with non-decreasing `from` only at points where no copy is in flight
// that the caller must not wait for (the byte load is waited on with the others).
struct BlockWalk {
    const uint8_t *row;
    int n, wbase = -64, wv = 0;
    uint64_t wm = 0;
    __device__ BlockWalk(const uint8_t *r, int count) : row(r), n(count) {}
    // first non-empty tile >= from (n if none); its class goes to val
    __device__ __forceinline__ int next(int from, int lane, int &val) {
        while (from < n) {
            if (from >= wbase + 64) {
                wbase = from & ~63;
                const int t = wbase + lane;
                wv = t < n ? (int)row[t] : 0;
                wm = __builtin_amdgcn_ballot_w64(wv != 0);
            }
            const uint64_t m = wm & (~0ull << (from - wbase));
            if (m) {
                const int off = (int)__builtin_ctzll(m);
                val = __builtin_amdgcn_readlane(wv, off);
                return wbase + off;
            }
            from = wbase + 64;
        }
        val = 0;
        return n;
    }
};

}  // namespace mm
