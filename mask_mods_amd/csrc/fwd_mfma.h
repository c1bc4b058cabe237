// fwd_mfma.h -- flash-attention forward for gfx950 with flex mods (bf16 / f16 inputs).
//
// One workgroup = 4 waves = 128 query rows of one (batch, query head); each wave owns
// 32 rows. Keys/values stream through LDS in tiles of 64, double buffered, with the
// next tile's global loads in flight while the current tile is computed.
//
// Both products run on the 32x32x16 MFMA with fp32 accumulation, in transposed form
// so that a lane always owns one query row:
//   S^T[j][i] = sum_d K[j][d] Q[i][d]      A = K tile from LDS, B = Q^T kept in VGPRs
//   O^T[d][i] += sum_j V^T[d][j] P^T[j][i] A = V^T tile from LDS, B = P^T from registers
// In the C layout a lane holds column i = lane % 32 and 16 rows, so the softmax
// reductions over keys are lane-local plus one exchange with lane ^ 32, and the
// per-row rescale of O is a per-lane scalar multiply.
//
// The contraction index of P^T V^T (the key) may be permuted freely as long as both
// operands agree; V^T is written to LDS with its keys in the order the S^T
// accumulator hands them to each lane, so P^T needs no data movement at all.
//
// Scores are kept in base-2 units (t = scale*log2(e)*q.k [+ slope*log2(e)*(j-i)]), so
// the softmax uses the hardware exp2. Semantics (FlyDSL PR #931, Summary): the
// score_mod sees the scaled score, the mask_mod is applied after it, and rows with no
// kept key produce O = 0, LSE = -inf (running max clamped to 0 while it is -inf, and
// a guarded 1/l in the epilogue).
#pragma once

#include "common.h"
#include "kernels.h"

namespace mm {

template <typename TT, int D, bool ALIBI, int MASK>
__global__ __launch_bounds__(256) void fwd_mfma_kernel(FwdParams p) {
    constexpr int BM = kFwdBM, BN = 64;
    constexpr int KS = D / 16;   // k-steps of Q K^T
    constexpr int DB = D / 32;   // 32-row blocks of O^T
    constexpr int NKB = BN / 32; // 32-key blocks of S^T per tile
    constexpr int KLD = D + 8;   // K tile row stride (elements), padded against bank conflicts
    constexpr int VLD = BN + 8;  // V^T tile row stride (elements)
    constexpr int TILE = BN * KLD + D * VLD;
    constexpr int KCH = BN * D / 8 / 256;     // 16-byte K chunks per thread per tile
    constexpr int VUNITS = (BN / 4) * (D / 8); // 4-key x 8-dim V blocks per tile
    typedef typename TT::vec8 V8;
    static_assert(KCH >= 1 && VUNITS <= 256, "tile shape");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    int L = xcd_remap(blockIdx.x, gridDim.x);
    const int qt_idx = L % p.n_qtiles;
    L /= p.n_qtiles;
    const int h = L % p.Hq;
    const int b = L / p.Hq;
    // causal: the last query tiles carry the most keys; start them first
    const int qt = (MASK & MASK_CAUSAL) ? (p.n_qtiles - 1 - qt_idx) : qt_idx;
    const int q0 = qt * BM;
    const int hk = h / p.group;

    const uint16_t *qg = (const uint16_t *)p.q + b * p.q_sb + h * p.q_sh;
    const uint16_t *kg = (const uint16_t *)p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vg = (const uint16_t *)p.v + b * p.v_sb + hk * p.v_sh;

    const int r0 = q0 + wave * 32;  // first row of this wave
    const int row = r0 + l32;       // the row this lane owns

    // Q^T fragments (B operand): row `row`, dims 16*ks + 8*hi .. +7
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

    // key range this workgroup can see
    const int row_max = min(q0 + BM, p.Sq) - 1;
    int j_lo = 0, j_hi = p.Skv;
    if (MASK & MASK_CAUSAL) j_hi = min(j_hi, row_max + 1);
    if (MASK & MASK_WINDOW) {
        j_lo = max(0, q0 - p.window);
        if (!(MASK & MASK_CAUSAL)) j_hi = min(j_hi, row_max + p.window + 1);
    }
    const int kt_lo = j_lo / BN;
    const int kt_hi = j_hi > j_lo ? (j_hi + BN - 1) / BN : kt_lo;

    float slope2 = 0.f;
    if (ALIBI) slope2 = (p.slopes ? p.slopes[h] : exp2f(-8.f * (float)(h + 1) / (float)p.Hq)) * kLog2e;

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // ---- global -> registers -> LDS staging ----
    u32x4 kreg[KCH];
    u32x4 vreg[4];
    auto load_tile = [&](int kt) {
        const int k0 = kt * BN;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = tid + 256 * c;
            const int j = idx / (D / 8), dc = idx % (D / 8);
            const int jj = k0 + j;
            kreg[c] = jj < p.Skv ? *(const u32x4 *)(kg + (int64_t)jj * p.k_ss + 8 * dc) : u32x4{0, 0, 0, 0};
        }
        if (tid < VUNITS) {
            const int kgi = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int jj = k0 + 4 * kgi + r;
                vreg[r] = jj < p.Skv ? *(const u32x4 *)(vg + (int64_t)jj * p.v_ss + 8 * dc) : u32x4{0, 0, 0, 0};
            }
        }
    };
    auto store_tile = [&](int buf) {
        uint16_t *Ks = smem + buf * TILE;
        uint16_t *Vt = Ks + BN * KLD;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = tid + 256 * c;
            const int j = idx / (D / 8), dc = idx % (D / 8);
            *(u32x4 *)(Ks + j * KLD + 8 * dc) = kreg[c];
        }
        if (tid < VUNITS) {
            const int kgi = tid / (D / 8), dc = tid % (D / 8);
            // within each 16-key block, 4-key groups 0,1,2,3 go to slots 0,2,1,3
            const int g = kgi & 3;
            const int pos = 16 * (kgi >> 2) + 4 * (((g & 1) << 1) | (g >> 1));
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1, sh = (e & 1) * 16;
                const uint32_t a0 = (vreg[0][w] >> sh) & 0xFFFFu, a1 = (vreg[1][w] >> sh) & 0xFFFFu;
                const uint32_t a2 = (vreg[2][w] >> sh) & 0xFFFFu, a3 = (vreg[3][w] >> sh) & 0xFFFFu;
                *(u32x2 *)(Vt + (8 * dc + e) * VLD + pos) = u32x2{a0 | (a1 << 16), a2 | (a3 << 16)};
            }
        }
    };

    if (kt_lo < kt_hi) {
        load_tile(kt_lo);
        store_tile(0);
    }
    __syncthreads();

    for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int buf = (kt - kt_lo) & 1;
        const bool more = kt + 1 < kt_hi;
        if (more) load_tile(kt + 1);

        const int k0 = kt * BN;
        const int r_last = r0 + 31;
        bool skip = false, need_mask = k0 + BN > p.Skv;
        if (MASK & MASK_CAUSAL) {
            skip |= k0 > r_last;
            need_mask |= k0 + BN - 1 > r0;
        }
        if (MASK & MASK_WINDOW) {
            skip |= (k0 - r_last > p.window) || (r0 - (k0 + BN - 1) > p.window);
            need_mask |= max(r_last - k0, k0 + BN - 1 - r0) > p.window;
        }

        if (!skip) {
            const uint16_t *Ks = smem + buf * TILE;
            const uint16_t *Vt = Ks + BN * KLD;
            f32x16 sacc[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                sacc[kb] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const V8 a = as_vec<V8>(*(const u32x4 *)(Ks + (32 * kb + l32) * KLD + 16 * ks + 8 * hi));
                    sacc[kb] = mfma32x32x16(a, qf[ks], sacc[kb]);
                }
            }
            // scale, score_mod, mask_mod; lane's keys: k0 + 32*kb + 8*(e/4) + 4*hi + e%4
            float mloc = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = k0 + 32 * kb + 8 * (e >> 2) + 4 * hi + (e & 3);
                    float t = sacc[kb][e] * p.scale_log2;
                    if (ALIBI) t += slope2 * (float)(j - row);
                    if (need_mask) {
                        bool keep = j < p.Skv;
                        if (MASK & MASK_CAUSAL) keep &= j <= row;
                        if (MASK & MASK_WINDOW) keep &= abs(row - j) <= p.window;
                        t = keep ? t : -INFINITY;
                    }
                    sacc[kb][e] = t;
                    mloc = fmaxf(mloc, t);
                }
            }
            mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
            const float m_new = fmaxf(m_run, mloc);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;  // clamp: no (-inf) - (-inf)
            const float alpha = fast_exp2(m_run - m_use);
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float pv = fast_exp2(sacc[kb][e] - m_use);
                    sacc[kb][e] = pv;
                    psum += pv;
                }
            }
            l_run = l_run * alpha + psum;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            // O^T += V^T P^T
#pragma unroll
            for (int ks = 0; ks < BN / 16; ++ks) {
                const f32x16 &s = sacc[ks >> 1];
                const int o8 = 8 * (ks & 1);
                const f32x8 pf32 = {s[o8 + 0], s[o8 + 1], s[o8 + 2], s[o8 + 3],
                                    s[o8 + 4], s[o8 + 5], s[o8 + 6], s[o8 + 7]};
                const V8 pf = cvt8(pf32, TT{});
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const V8 a = as_vec<V8>(*(const u32x4 *)(Vt + (32 * db + l32) * VLD + 16 * ks + 8 * hi));
                    oacc[db] = mfma32x32x16(a, pf, oacc[db]);
                }
            }
        }
        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
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
hipError_t launch_fwd_mfma(const FwdParams &p, bool alibi, int mask, hipStream_t s) {
    const dim3 grid((unsigned)(p.n_qtiles * p.Hq * p.B)), block(256);
#define MM_FWD_CASE(A, M) \
    case (A) * 4 + (M): fwd_mfma_kernel<TT, D, (A) != 0, (M)><<<grid, block, 0, s>>>(p); break;
    switch ((alibi ? 4 : 0) + (mask & 3)) {
        MM_FWD_CASE(0, 0)
        MM_FWD_CASE(0, 1)
        MM_FWD_CASE(0, 2)
        MM_FWD_CASE(0, 3)
        MM_FWD_CASE(1, 0)
        MM_FWD_CASE(1, 1)
        MM_FWD_CASE(1, 2)
        MM_FWD_CASE(1, 3)
    }
#undef MM_FWD_CASE
    return hipGetLastError();
}

}  // namespace mm
