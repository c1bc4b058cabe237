// fwd_f32.hip -- fp32-input forward attention on the vector ALUs.
//
// The correctness path for fp32 tensors (no performance target): one thread owns one
// query row, keeps q and the output accumulator in registers and streams every
// visible key with an online softmax in fp32. Same semantics and mask handling as the
// MFMA path: scale, then score_mod, then mask_mod (and the block mask); fully masked
// rows give 0 / -inf.
#include "common.h"
#include "kernels.h"

namespace mm {

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdParams p, int alibi, int mask) {
    const int64_t rid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nrows = (int64_t)p.B * p.Hq * p.Sq;
    if (rid >= nrows) return;
    const int row = (int)(rid % p.Sq);
    const int h = (int)((rid / p.Sq) % p.Hq);
    const int b = (int)(rid / ((int64_t)p.Sq * p.Hq));
    const int hk = h / p.group;

    const float *qr = (const float *)p.q + b * p.q_sb + h * p.q_sh + (int64_t)row * p.q_ss;
    const float *kg = (const float *)p.k + b * p.k_sb + hk * p.k_sh;
    const float *vg = (const float *)p.v + b * p.v_sb + hk * p.v_sh;

    float q[D], o[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = qr[d] * p.scale_log2;
        o[d] = 0.f;
    }
    const float slope2 = alibi ? (p.slopes ? p.slopes[h] : exp2f(-8.f * (float)(h + 1) / (float)p.Hq)) * kLog2e : 0.f;

    // with a block mask, full blocks bypass the predicates: test each key instead of
    // narrowing the range
    const uint8_t *bm_row = p.bm ? p.bm + b * p.bm_sb + h * p.bm_sh + (int64_t)(row / kBlockQ) * p.bm_sq : nullptr;
    int j_lo = 0, j_hi = p.Skv;
    if ((mask & MASK_CAUSAL) && !bm_row) j_hi = min(j_hi, row + 1);
    if ((mask & MASK_WINDOW) && !bm_row) {
        j_lo = max(j_lo, row - p.window);
        j_hi = min(j_hi, row + p.window + 1);
    }
    const int32_t *kd = (mask & MASK_DOC) ? p.kvdoc + b * p.kvdoc_sb : nullptr;
    const int mydoc = kd ? p.qdoc[b * p.qdoc_sb + row] : 0;
    if (kd && !bm_row) {
        j_lo = max(j_lo, doc_lower(kd, p.Skv, mydoc));
        j_hi = min(j_hi, doc_upper(kd, p.Skv, mydoc));
    }
    bool dropped = false;
    if (p.rowdrop) dropped = fmix32(p.rd_seed ^ (uint32_t)rid) < p.rd_thr;
    if (dropped) j_hi = j_lo;

    float m = -INFINITY, l = 0.f;
    for (int j = j_lo; j < j_hi; ++j) {
        if (bm_row) {
            const int blk = bm_row[j / kBlockKV];
            if (blk == 0) continue;
            if (blk == 1 && (mask & MASK_CAUSAL) && j > row) continue;
            if (blk == 1 && (mask & MASK_WINDOW) && abs(row - j) > p.window) continue;
            if (blk == 1 && kd && kd[j] != mydoc) continue;
        }
        const float *kr = kg + (int64_t)j * p.k_ss;
        float t = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) t = fmaf(q[d], kr[d], t);
        if (alibi) t += slope2 * (float)(j - row);
        const float m_new = fmaxf(m, t);
        const float alpha = fast_exp2(m - m_new);
        const float pv = fast_exp2(t - m_new);
        l = l * alpha + pv;
        const float *vr = vg + (int64_t)j * p.v_ss;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = fmaf(pv, vr[d], o[d] * alpha);
        m = m_new;
    }
    const bool live = l > 0.f;
    const float inv = live ? 1.f / l : 0.f;
    float *orow = (float *)p.o + b * p.o_sb + h * p.o_sh + (int64_t)row * p.o_ss;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = o[d] * inv;
    if (p.lse) p.lse[rid] = live ? (m + __log2f(l)) * kLn2 : -INFINITY;
}

hipError_t launch_fwd_f32(const FwdParams &p, int D, bool alibi, int mask, hipStream_t s) {
    const int64_t nrows = (int64_t)p.B * p.Hq * p.Sq;
    const dim3 grid((unsigned)((nrows + 63) / 64)), block(64);
    if (D == 64)
        fwd_f32_kernel<64><<<grid, block, 0, s>>>(p, alibi, mask);
    else
        fwd_f32_kernel<128><<<grid, block, 0, s>>>(p, alibi, mask);
    return hipGetLastError();
}

}  // namespace mm
