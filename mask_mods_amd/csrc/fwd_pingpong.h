// fwd_pingpong.h -- flash-attention forward, 8-wave "ping-pong" schedule (gfx950).
//
// Same arithmetic, operand layouts and LDS tile format as fwd_mfma_kernel (see
// fwd_mfma.h), organised so the two waves that share a SIMD alternate between the
// MFMA-heavy and the VALU-heavy part of the loop instead of meeting by chance.
//
// A workgroup is 8 waves = 256 query rows of one (batch, head): group 0 is waves 0-3
// (rows q0 .. q0+127), group 1 is waves 4-7 (rows q0+128 ..); wave w and wave w+4 run
// on the same SIMD. Work per key tile i splits into
//   MFMA step i : O += V_{i-1} P_{i-1} (previous tile), then S_i = K_i Q^T
//   VALU step i : softmax of S_i -> P_i (max, lazy rescale, exp2, row sum)
// and the workgroup advances in phases separated by barriers. In every phase one group
// runs an MFMA step while the other runs a VALU step; group 1 lags group 0 by one phase:
//   phase 4m   : group 0 MFMA(2m)   [K buf0, V buf1]   group 1 VALU(2m-1)
//   phase 4m+1 : group 1 MFMA(2m)   [K buf0, V buf1]   group 0 VALU(2m)
//   phase 4m+2 : group 0 MFMA(2m+1) [K buf1, V buf0]   group 1 VALU(2m)
//   phase 4m+3 : group 1 MFMA(2m+1) [K buf1, V buf0]   group 0 VALU(2m+1)
// K_i lives in K buf (i%2) during phases 2i, 2i+1 and V_i in V buf (i%2) during 2i+2,
// 2i+3. At every even phase 2j all waves issue the DMA of K_{j+1} and V_j into the
// buffers freed in phase 2j-1, and wait for it before the barrier that ends phase 2j+1,
// so each copy has two phases to land. Buffer choice is static in every phase.
#pragma once

#include "fwd_mfma.h"

namespace mm {

// barrier that also drains this wave's LDS reads (and, with VM, its DMA copies)
template <bool VM>
__device__ __forceinline__ void pp_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (VM)
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    else
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
}

template <typename TT, int D, bool ALIBI, int MASK>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pp_kernel(FwdParams p) {
    constexpr int BM = 256, BN = 64;
    constexpr int KS = D / 16, DB = D / 32, NKB = BN / 32;
    typedef Tile<D> TL;
    constexpr int TILEB = BN * TL::ROWB;
    constexpr int BLKS = TILEB / 1024;  // 1 KB DMA blocks per tile
    constexpr int LOADS = BLKS / 8;     // per wave per tile
    constexpr int RPI = 1024 / TL::ROWB;
    constexpr float kRescale = 8.f;
    typedef typename TT::vec8 V8;
    static_assert(LOADS >= 1 && LOADS * 8 == BLKS, "tile shape");

    __shared__ __attribute__((aligned(1024))) unsigned char kbuf0[TILEB], vbuf0[TILEB];
    __shared__ __attribute__((aligned(1024))) unsigned char kbuf1[TILEB], vbuf1[TILEB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int grp = wave_s >> 2;

    int L = xcd_remap(blockIdx.x, gridDim.x);
    const int qt_idx = L % p.n_qtiles;
    L /= p.n_qtiles;
    const int h = L % p.Hq;
    const int b = L / p.Hq;
    const int qt = (MASK & MASK_CAUSAL) ? (p.n_qtiles - 1 - qt_idx) : qt_idx;
    const int q0 = qt * BM;
    const int hk = h / p.group;

    const uint16_t *qg = (const uint16_t *)p.q + b * p.q_sb + h * p.q_sh;
    const uint16_t *kg = (const uint16_t *)p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vg = (const uint16_t *)p.v + b * p.v_sb + hk * p.v_sh;

    const int r0 = q0 + wave_s * 32;
    const int row = r0 + l32;

    V8 qf[KS];
    {
        const bool ok = row < p.Sq;
        const uint16_t *qr = qg + (int64_t)(ok ? row : 0) * p.q_ss + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 x = ok ? *(const u32x4 *)(qr + 16 * ks) : u32x4{0, 0, 0, 0};
            qf[ks] = as_vec<V8>(x);
        }
    }

    const int row_max = min(q0 + BM, p.Sq) - 1;
    int j_lo = 0, j_hi = p.Skv;
    if (MASK & MASK_CAUSAL) j_hi = min(j_hi, row_max + 1);
    if (MASK & MASK_WINDOW) {
        j_lo = max(0, q0 - p.window);
        if (!(MASK & MASK_CAUSAL)) j_hi = min(j_hi, row_max + p.window + 1);
    }
    const int kt_lo = j_lo / BN;
    const int n = j_hi > j_lo ? (j_hi + BN - 1) / BN - kt_lo : 0;  // key tiles to visit

    float slope2 = 0.f;
    if (ALIBI) slope2 = (p.slopes ? p.slopes[h] : exp2f(-8.f * (float)(h + 1) / (float)p.Hq)) * kLog2e;
    const float c2 = p.scale_log2;

    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = TL::off(l32, 2 * ks + hi);
    int voff[DB][2];
    {
        const int G = lane >> 4, t = lane & 15;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int m2 = 0; m2 < 2; ++m2) {
                const int r = 8 * m2 + 4 * hi + (t >> 2);
                const int d = 32 * db + 16 * (G & 1) + 4 * (t & 3);
                voff[db][m2] = TL::off(r, d >> 3) + 2 * (d & 7);
            }
    }

    // DMA: wave w copies blocks w*LOADS .. of each tile (see fwd_mfma.h for the mapping)
    uint32_t kgo[LOADS], vgo[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int r = (wave_s * LOADS + i) * RPI + lane / TL::CH;
        const int c = (lane % TL::CH) ^ TL::swz(r);
        kgo[i] = (uint32_t)(r * (int)p.k_ss + 8 * c) * 2u;
        vgo[i] = (uint32_t)(r * (int)p.v_ss + 8 * c) * 2u;
    }
    auto dma = [&](int ti, const uint16_t *g, int64_t ss, const uint32_t *go, unsigned char *dst) {
        const int k0 = (kt_lo + ti) * BN;
        if (k0 + BN <= p.Skv) {
            const char *base = (const char *)(g + (int64_t)k0 * ss);
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                __builtin_amdgcn_global_load_lds((const void *)(base + go[i]),
                                                 (MM_LDS void *)(dst + (wave_s * LOADS + i) * 1024), 16, 0, 0);
        } else {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int r = (wave_s * LOADS + i) * RPI + lane / TL::CH;
                const int c = (lane % TL::CH) ^ TL::swz(r);
                const int gr = min(k0 + r, p.Skv - 1);
                __builtin_amdgcn_global_load_lds((const void *)(g + (int64_t)gr * ss + 8 * c),
                                                 (MM_LDS void *)(dst + (wave_s * LOADS + i) * 1024), 16, 0, 0);
            }
        }
    };

    // per-wave tile classification (rows r0 .. r0+31 against keys k0 .. k0+63)
    auto classify = [&](int ti, bool &skip, bool &need_mask) {
        const int k0 = (kt_lo + ti) * BN;
        const int r_last = r0 + 31;
        skip = false;
        need_mask = k0 + BN > p.Skv;
        if (MASK & MASK_CAUSAL) {
            skip |= k0 > r_last;
            need_mask |= k0 + BN - 1 > r0;
        }
        if (MASK & MASK_WINDOW) {
            skip |= (k0 - r_last > p.window) || (r0 - (k0 + BN - 1) > p.window);
            need_mask |= max(r_last - k0, k0 + BN - 1 - r0) > p.window;
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    f32x16 sacc[NKB];
    uint32_t pp[NKB][8];
    float m_run = -INFINITY, l_run = 0.f;

    // MFMA step i: O += V_{i-1} P_{i-1}, then S_i = K_i Q^T
    auto mfma_step = [&](int i, const unsigned char *Kt, const unsigned char *Vt) {
        bool skip, nm_;
        MM_PRIO_HI();
        if (i >= 1 && i - 1 < n) {
            classify(i - 1, skip, nm_);
            if (!skip) {
#pragma unroll
                for (int ks = 0; ks < BN / 16; ++ks) {
                    const int kb = ks >> 1, o4 = 4 * (ks & 1);
                    const V8 pf = as_vec<V8>(u32x4{pp[kb][o4], pp[kb][o4 + 1], pp[kb][o4 + 2], pp[kb][o4 + 3]});
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (MM_LDS s16x4 *)(Vt + ks * 16 * TL::ROWB + voff[db][0]));
                        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (MM_LDS s16x4 *)(Vt + ks * 16 * TL::ROWB + voff[db][1]));
                        const u32x2 a0 = __builtin_bit_cast(u32x2, lo), a1 = __builtin_bit_cast(u32x2, hi4);
                        const V8 a = as_vec<V8>(u32x4{a0[0], a0[1], a1[0], a1[1]});
                        oacc[db] = mfma32x32x16(a, pf, oacc[db]);
                    }
                }
            }
        }
        if (i < n) {
            classify(i, skip, nm_);
            if (!skip) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    sacc[kb] = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const V8 a = as_vec<V8>(*(const u32x4 *)(Kt + kb * 32 * TL::ROWB + koff[ks]));
                        sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
                    }
                }
            }
        }
        MM_PRIO_LO();
    };

    // VALU step i: scale, mods, masks, online softmax of S_i into P_i
    auto valu_step = [&](int i) {
        if (i < 0 || i >= n) return;
        bool skip, need_mask;
        classify(i, skip, need_mask);
        if (skip) return;
        const int k0 = (kt_lo + i) * BN;
        float mloc = -INFINITY, cc;
        const bool general = ALIBI || need_mask || !(c2 > 0.f);
        if (general) {
            const float base = ALIBI ? slope2 * (float)(k0 + 4 * hi - row) : 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jo = 32 * kb + 8 * (e >> 2) + (e & 3);
                    float t = ALIBI ? fmaf(sacc[kb][e], c2, fmaf(slope2, (float)jo, base)) : sacc[kb][e] * c2;
                    if (need_mask) {
                        const int j = k0 + 4 * hi + jo;
                        bool keep = j < p.Skv;
                        if (MASK & MASK_CAUSAL) keep &= j <= row;
                        if (MASK & MASK_WINDOW) keep &= abs(row - j) <= p.window;
                        t = keep ? t : -INFINITY;
                    }
                    sacc[kb][e] = t;
                    mloc = fmaxf(mloc, t);
                }
            }
            cc = 1.f;
        } else {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sacc[kb][e]);
            mloc *= c2;
            cc = c2;
        }
        mloc = row_max2(mloc);
        if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescale)) {
            const float m_new = fmaxf(m_run, mloc);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
        const float nm = m_run == -INFINITY ? 0.f : -m_run;
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float x0 = fast_exp2(fmaf(sacc[kb][2 * e2], cc, nm));
                const float x1 = fast_exp2(fmaf(sacc[kb][2 * e2 + 1], cc, nm));
                pp[kb][e2] = pack2(x0, x1, TT{});
                psum = dot2_ones(pp[kb][e2], psum, TT{});
            }
        l_run += psum;
    };

    if (n > 0) dma(0, kg, p.k_ss, kgo, kbuf0);
    pp_barrier<true>();
    // Each group runs its own straight-line loop over blocks of four phases; both loops
    // execute the same barriers in the same order, so the two groups stay one phase
    // apart. DMA at even phases 2j: K_{j+1} and V_j into the buffers freed at 2j-1.
    const int blocks = (2 * n + 2 + 3) / 4;
    if (grp == 0) {
        for (int it = 0; it < blocks; ++it) {
            const int i0 = 2 * it;
            if (i0 + 1 < n) dma(i0 + 1, kg, p.k_ss, kgo, kbuf1);
            if (i0 < n) dma(i0, vg, p.v_ss, vgo, vbuf0);
            mfma_step(i0, kbuf0, vbuf1);
            pp_barrier<false>();
            valu_step(i0);
            pp_barrier<true>();
            if (i0 + 2 < n) dma(i0 + 2, kg, p.k_ss, kgo, kbuf0);
            if (i0 + 1 < n) dma(i0 + 1, vg, p.v_ss, vgo, vbuf1);
            mfma_step(i0 + 1, kbuf1, vbuf0);
            pp_barrier<false>();
            valu_step(i0 + 1);
            pp_barrier<true>();
        }
    } else {
        for (int it = 0; it < blocks; ++it) {
            const int i0 = 2 * it;
            if (i0 + 1 < n) dma(i0 + 1, kg, p.k_ss, kgo, kbuf1);
            if (i0 < n) dma(i0, vg, p.v_ss, vgo, vbuf0);
            valu_step(i0 - 1);
            pp_barrier<false>();
            mfma_step(i0, kbuf0, vbuf1);
            pp_barrier<true>();
            if (i0 + 2 < n) dma(i0 + 2, kg, p.k_ss, kgo, kbuf0);
            if (i0 + 1 < n) dma(i0 + 1, vg, p.v_ss, vgo, vbuf1);
            valu_step(i0);
            pp_barrier<false>();
            mfma_step(i0 + 1, kbuf1, vbuf0);
            pp_barrier<true>();
        }
    }

    // ---- epilogue (as in fwd_mfma_kernel) ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    bool dropped = false;
    if (p.rowdrop) {
        const uint32_t rid = (uint32_t)(((int64_t)b * p.Hq + h) * p.Sq + row);
        dropped = fmix32(p.rd_seed ^ rid) < p.rd_thr;
    }
    const bool live = l_tot > 0.f && !dropped;
    const float inv = live ? 1.f / l_tot : 0.f;
    if (row < p.Sq) {
        uint16_t *og = (uint16_t *)p.o + b * p.o_sb + h * p.o_sh + (int64_t)row * p.o_ss;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 x = {oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv,
                                 oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
                *(typename TT::vec4 *)(og + 32 * db + 8 * g4 + 4 * hi) = cvt4(x, TT{});
            }
        }
        if (hi == 0 && p.lse) {
            p.lse[((int64_t)b * p.Hq + h) * p.Sq + row] = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <typename TT, int D>
hipError_t launch_fwd_pp(FwdParams p, bool alibi, int mask, hipStream_t s) {
    p.n_qtiles = (p.Sq + 255) / 256;
    const dim3 grid((unsigned)(p.n_qtiles * p.Hq * p.B)), block(512);
#define MM_PP_CASE(A, M) \
    case (A) * 4 + (M): fwd_pp_kernel<TT, D, (A) != 0, (M)><<<grid, block, 0, s>>>(p); break;
    switch ((alibi ? 4 : 0) + (mask & 3)) {
        MM_PP_CASE(0, 0)
        MM_PP_CASE(0, 1)
        MM_PP_CASE(0, 2)
        MM_PP_CASE(0, 3)
        MM_PP_CASE(1, 0)
        MM_PP_CASE(1, 1)
        MM_PP_CASE(1, 2)
        MM_PP_CASE(1, 3)
    }
#undef MM_PP_CASE
    return hipGetLastError();
}

}  // namespace mm
