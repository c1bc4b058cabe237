// block_mask.hip -- block-mask classes for the built-in mask_mods.
//
// The counterpart of building a BlockMask from a mask_mod: for every (query block,
// key block) the kernel classifies the block as empty (no pair kept), full (every
// pair kept) or partial, for the causal and sliding-window predicates. Both
// predicates depend only on d = q_idx - kv_idx (causal keeps d >= 0, the window keeps
// -w <= d <= w), and over a rectangle of pairs d takes every integer between its
// extremes, so two comparisons per block decide the class exactly. Pairs outside
// q_idx < Sq, kv_idx < Skv do not count.
#include "common.h"
#include "kernels.h"

namespace mm {

__global__ __launch_bounds__(256) void block_mask_kernel(uint8_t *out, int64_t ld, int nqb, int nkb, int Sq,
                                                         int Skv, int64_t d_lo, int64_t d_hi) {
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= (int64_t)nqb * nkb) return;
    const int qb = (int)(idx / nkb), kb = (int)(idx % nkb);
    const int64_t i0 = (int64_t)qb * kBlockQ, i1 = min((int64_t)Sq, i0 + kBlockQ) - 1;
    const int64_t j0 = (int64_t)kb * kBlockKV, j1 = min((int64_t)Skv, j0 + kBlockKV) - 1;
    const int64_t dmin = i0 - j1, dmax = i1 - j0;
    uint8_t cls;
    if (dmax < d_lo || dmin > d_hi) cls = 0;
    else if (dmin >= d_lo && dmax <= d_hi) cls = 2;
    else cls = 1;
    out[(int64_t)qb * ld + kb] = cls;
}

hipError_t launch_block_mask(uint8_t *out, int64_t ld, int Sq, int Skv, bool causal, int window,
                             hipStream_t s) {
    const int nqb = (Sq + kBlockQ - 1) / kBlockQ, nkb = (Skv + kBlockKV - 1) / kBlockKV;
    const int64_t n = (int64_t)nqb * nkb;
    if (n == 0) return hipSuccess;
    // the admitted range of d = q_idx - kv_idx
    int64_t d_lo = INT64_MIN / 2, d_hi = INT64_MAX / 2;
    if (causal) d_lo = 0;
    if (window >= 0) {
        d_lo = d_lo > -(int64_t)window ? d_lo : -(int64_t)window;
        d_hi = window;
    }
    block_mask_kernel<<<dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s>>>(out, ld, nqb, nkb, Sq, Skv, d_lo,
                                                                              d_hi);
    return hipGetLastError();
}

}  // namespace mm
