// bwd.h -- attention backward for gfx950 (bf16 / f16): dQ, dK, dV with the flex mods.
//
// For kept pairs, with P = exp(s - LSE) recomputed from the forward's LSE,
//   dV_j = sum_i P_ij dO_i,   dP_ij = dO_i . V_j,   dS_ij = P_ij (dP_ij - D_i),
//   dQ_i = scale sum_j dS_ij K_j,   dK_j = scale sum_i dS_ij Q_i,   D_i = dO_i . O_i.
// Masked pairs, and rows with no kept key (LSE = -inf, which covers the row-drop mod),
// contribute nothing. Three launches, no atomics:
//   bwd_pre_kernel    D_i and LSE_i in base 2 (+inf for dead rows, so P = 2^(t - lse2) = 0)
//   bwd_dq_kernel     shaped like the forward: a lane owns one query row; per 64-key tile
//                     S^T = K Q^T and dP^T = V dO^T (A = K / V rows from LDS, B = Q^T / dO^T
//                     held in VGPRs), then dQ^T += K^T dS^T (K^T by transpose reads, dS^T
//                     from registers in the accumulator's key order)
//   bwd_dkdv_kernel   a lane owns one key: per 64-row tile of Q and dO staged in LDS,
//                     S = Q K^T and dP = dO V^T (B = K^T / V^T held in VGPRs), then
//                     dV += P^T dO and dK += dS^T Q with dO^T / Q^T by transpose reads and
//                     P^T / dS^T from registers; the loop runs over every query head of
//                     the kv head's GQA group, so dK and dV are complete in one workgroup.
// The tiles use the forward's swizzled layout and DMA copies (fwd_mfma.h, fwd_common.h).
#pragma once

#include "fwd_mfma.h"

namespace mm {

// ---- -D_i = -(dO_i . O_i) and lse2_i = LSE_i * log2(e) (+inf when LSE_i = -inf) ----
// (-D: the dK/dV kernel starts its dP accumulators at it, so its MFMAs give dP - D)
template <typename TT, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdParams p) {
    constexpr int LPR = D / 8;  // lanes per row, 8 elements each
    const int64_t nrows = (int64_t)p.B * p.Hq * p.Sq;
    const int64_t rid = (int64_t)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (rid < nrows) {
        const int i = (int)(rid % p.Sq);
        const int h = (int)((rid / p.Sq) % p.Hq);
        const int b = (int)(rid / ((int64_t)p.Sq * p.Hq));
        const uint16_t *orow = (const uint16_t *)p.o + b * p.o_sb + h * p.o_sh + (int64_t)i * p.o_ss;
        const uint16_t *drow = (const uint16_t *)p.dout + b * p.do_sb + h * p.do_sh + (int64_t)i * p.do_ss;
        const f32x8 ov = widen8(*(const u32x4 *)(orow + 8 * c), TT{});
        const f32x8 dv = widen8(*(const u32x4 *)(drow + 8 * c), TT{});
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(ov[e], dv[e], acc);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (rid < nrows && c == 0) {
        const int64_t w = (rid / p.Sq) * p.sq_pad + rid % p.Sq;
        p.ws_nd[w] = -acc;
        const float l = p.lse[rid];
        p.ws_lse2[w] = l == -INFINITY ? INFINITY : l * kLog2e;
    }
}

// ---- dQ: one workgroup = NW waves x 32 query rows of one (b, h) ----
template <typename TT, int D, bool ALIBI, int MASK, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdParams p) {
    constexpr int BM = 32 * NW, BN = 64;
    constexpr int KS = D / 16, DB = D / 32, NKB = BN / 32;
    typedef Tile<D> TL;
    constexpr int TILEB = BN * TL::ROWB;
    constexpr int LOADS = TILEB / 1024 / NW;
    constexpr int RPI = 1024 / TL::ROWB;
    typedef typename TT::vec8 V8;
    static_assert(LOADS >= 1 && LOADS * NW * 1024 == TILEB, "tile shape");

    // with the document mask a stage also holds its tile's 64 key document ids, so that
    // the tile reads them from LDS (a global load inside the tile would make the compiler
    // wait for every copy in flight, the next tile's included)
    constexpr int DOCB = (MASK & MASK_DOC) ? 1024 : 0;
    __shared__ __attribute__((aligned(1024))) unsigned char kv0[2 * TILEB + DOCB];
    __shared__ __attribute__((aligned(1024))) unsigned char kv1[2 * TILEB + DOCB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    // causal: the last query tiles carry the most keys; they start first
    int qt, pair;
    work_item(blockIdx.x, gridDim.x, p.n_tiles, (MASK & MASK_CAUSAL) != 0, qt, pair);
    const int h = pair % p.Hq;
    const int b = pair / p.Hq;
    const int q0 = qt * BM;
    const int hk = h / p.group;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int r0 = q0 + wave_s * 32;
    const int row = r0 + l32;
    const bool row_ok = row < p.Sq;

    const uint16_t *kg = (const uint16_t *)p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vg = (const uint16_t *)p.v + b * p.v_sb + hk * p.v_sh;

    // Q^T and dO^T fragments (B operands): row `row`, dims 16*ks + 8*hi .. +7
    V8 qf[KS], df[KS];
    {
        const int rr = row_ok ? row : 0;
        const uint16_t *qr = (const uint16_t *)p.q + b * p.q_sb + h * p.q_sh + (int64_t)rr * p.q_ss + 8 * hi;
        const uint16_t *dr = (const uint16_t *)p.dout + b * p.do_sb + h * p.do_sh + (int64_t)rr * p.do_ss + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qf[ks] = as_vec<V8>(row_ok ? *(const u32x4 *)(qr + 16 * ks) : u32x4{0, 0, 0, 0});
            df[ks] = as_vec<V8>(row_ok ? *(const u32x4 *)(dr + 16 * ks) : u32x4{0, 0, 0, 0});
        }
    }
    const int64_t wid = ((int64_t)b * p.Hq + h) * p.sq_pad + (row_ok ? row : 0);
    const float lse2 = row_ok ? p.ws_lse2[wid] : INFINITY;
    const float ndr = row_ok ? p.ws_nd[wid] : 0.f;  // -D

    const int row_max = min(q0 + BM, p.Sq) - 1;
    int j_lo = 0, j_hi = p.Skv;
    if ((MASK & MASK_CAUSAL) && !(MASK & MASK_BLOCK)) j_hi = min(j_hi, row_max + 1);
    if ((MASK & MASK_WINDOW) && !(MASK & MASK_BLOCK)) {
        j_lo = max(0, q0 - p.window);
        if (!(MASK & MASK_CAUSAL)) j_hi = min(j_hi, row_max + p.window + 1);
    }
    // packed documents: keys of the documents of the tile's rows; per wave, the document
    // ids of its first and last rows and, per lane, of its row
    int wd_lo = 0, wd_hi = 0, mydoc = 0;
    if (MASK & MASK_DOC) {
        const int32_t *qd = p.qdoc + b * p.qdoc_sb, *kd = p.kvdoc + b * p.kvdoc_sb;
        if (!(MASK & MASK_BLOCK)) {
            int dlo, dhi;
            wave_search_range(kd, p.Skv, qd[q0], qd[row_max], lane, dlo, dhi);
            j_lo = max(j_lo, dlo);
            j_hi = min(j_hi, dhi);
        }
        wd_lo = qd[min(r0, p.Sq - 1)];
        wd_hi = qd[min(r0 + 31, p.Sq - 1)];
        mydoc = qd[min(row, p.Sq - 1)];
    }
    const int kt_lo = j_lo / BN;
    const int kt_hi = j_hi > j_lo ? (j_hi + BN - 1) / BN : kt_lo;

    float slope2 = 0.f;
    if (ALIBI) slope2 = (p.slopes ? p.slopes[h] : exp2f(-8.f * (float)(h + 1) / (float)p.Hq)) * kLog2e;
    const float c2 = p.scale_log2;

    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = TL::off(l32, 2 * ks + hi);
    int voff[DB][2];  // transposed reads of a tile (K^T here), as the forward's V^T
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
    uint32_t kgo[LOADS], vgo[LOADS];
    int trow[LOADS], tchunk[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int r = (wave_s * LOADS + i) * RPI + lane / TL::CH;
        const int c = (lane % TL::CH) ^ TL::swz(r);
        trow[i] = r;
        tchunk[i] = c;
        kgo[i] = (uint32_t)(r * (int)p.k_ss + 8 * c) * 2u;
        vgo[i] = (uint32_t)(r * (int)p.v_ss + 8 * c) * 2u;
    }
    auto load_tile = [&](int kt, unsigned char *kdst, unsigned char *vdst) {
        const int k0 = kt * BN;
        const uint32_t kl = lds_addr(kdst) + (uint32_t)(wave_s * LOADS) * 1024u;
        const uint32_t vl = lds_addr(vdst) + (uint32_t)(wave_s * LOADS) * 1024u;
        if ((MASK & MASK_DOC) && wave_s == 0) {
            // the tile's key document ids (clamped to the last key) after its V tile
            dma4_vaddr(p.kvdoc + b * p.kvdoc_sb + min(k0 + lane, p.Skv - 1), lds_addr(kdst) + 2 * TILEB);
        }
        if (k0 + BN <= p.Skv) {
            const char *kb = (const char *)(kg + (int64_t)k0 * p.k_ss);
            const char *vb = (const char *)(vg + (int64_t)k0 * p.v_ss);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                dma16_sbase(kb, kgo[i], kl + i * 1024);
                dma16_sbase(vb, vgo[i], vl + i * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int gr = min(k0 + trow[i], p.Skv - 1);
                dma16_vaddr(kg + (int64_t)gr * p.k_ss + 8 * tchunk[i], kl + i * 1024);
                dma16_vaddr(vg + (int64_t)gr * p.v_ss + 8 * tchunk[i], vl + i * 1024);
            }
        }
    };

    f32x16 dqacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) dqacc[db] = f32x16{};

    auto tile = [&](int kt, int blk, const unsigned char *Kt, const unsigned char *Vt, int next,
                    unsigned char *Kn, unsigned char *Vn) {
        if (next >= 0) load_tile(next, Kn, Vn);
        const int k0 = kt * BN;
        const int r_last = r0 + 31;
        const bool pred = blk == 1;
        bool skip = kt >= kt_hi, need_mask = k0 + BN > p.Skv;
        if ((MASK & MASK_CAUSAL) && pred) {
            skip |= k0 > r_last;
            need_mask |= k0 + BN - 1 > r0;
        }
        if ((MASK & MASK_WINDOW) && pred) {
            skip |= (k0 - r_last > p.window) || (r0 - (k0 + BN - 1) > p.window);
            need_mask |= max(r_last - k0, k0 + BN - 1 - r0) > p.window;
        }
        bool doc_mask = false;
        const int32_t *kd = (const int32_t *)(Kt + 2 * TILEB);  // the tile's key ids, clamped
        if ((MASK & MASK_DOC) && pred && !skip) {
            const int kdl = kd[0], kdh = kd[BN - 1];
            skip |= kdh < wd_lo || kdl > wd_hi;
            doc_mask = !(wd_lo == wd_hi && kdl == kdh && kdl == wd_lo);
            need_mask |= doc_mask;
        }
        if (skip) return;
        // a tile that straddles documents: the lane's document's keys, [dfirst, dend)
        int dfirst = 0, dend = BN;
        if ((MASK & MASK_DOC) && doc_mask) tile_doc_range(kd[lane], mydoc, dfirst, dend);
        // one 32-key block at a time: S^T = K Q^T and dP^T = V dO^T, then dS^T, then
        // dQ^T += K^T dS^T over the block's two 16-key k-steps
        const bool general = ALIBI || need_mask;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16 sacc = f32x16{}, dpacc = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 ka = *(const u32x4 *)(Kt + kb * 32 * TL::ROWB + koff[ks]);
                const u32x4 va = *(const u32x4 *)(Vt + kb * 32 * TL::ROWB + koff[ks]);
                sacc = mfma32x32x16(as_vec<V8>(ka), qf[ks], sacc);
                dpacc = mfma32x32x16(as_vec<V8>(va), df[ks], dpacc);
            }
            // P = 2^(t - lse2) and dS = P (dP - D) as 16-bit pairs, keys in accumulator order
            uint32_t dsp[8];
            // gen: scale and alibi applied to the score; masked: the predicates too (an
            // alibi tile that needs no mask takes gen without masked)
            // the lane's kept keys in this 32-key block: one interval of offsets jo = j -
            // k0 - 4*hi (each predicate keeps an interval)
            const int rel = row - k0 - 4 * hi;
            int jlo = 0, jhi = p.Skv - k0 - 4 * hi;
            if ((MASK & MASK_CAUSAL) && pred) jhi = min(jhi, rel + 1);
            if ((MASK & MASK_WINDOW) && pred) {
                jlo = max(jlo, rel - p.window);
                jhi = min(jhi, rel + p.window + 1);
            }
            if ((MASK & MASK_DOC) && pred) {
                jlo = max(jlo, dfirst - 4 * hi);
                jhi = min(jhi, dend - 4 * hi);
            }
            const uint32_t span = jhi > jlo ? (uint32_t)(jhi - jlo) : 0u;
            auto make_ds = [&](bool gen, bool masked) {
                const float base = ALIBI ? slope2 * (float)(k0 + 4 * hi - row) : 0.f;
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    float x[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int e = 2 * e2 + u;
                        const int jo = 32 * kb + 8 * (e >> 2) + (e & 3);
                        float pv;
                        if (gen) {
                            const float t = ALIBI ? fmaf(sacc[e], c2, fmaf(slope2, (float)jo, base)) : sacc[e] * c2;
                            const bool keep = !masked || (uint32_t)(jo - jlo) < span;
                            pv = keep ? fast_exp2(t - lse2) : 0.f;
                        } else {
                            pv = fast_exp2(fmaf(sacc[e], c2, -lse2));
                        }
                        x[u] = pv * (dpacc[e] + ndr);
                    }
                    dsp[e2] = pack2(x[0], x[1], TT{});
                }
            };
            if (ALIBI && !need_mask)
                make_ds(true, false);
            else if (general)
                make_ds(true, true);
            else
                make_ds(false, false);
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int ks = 2 * kb + half, o4 = 4 * half;
                const V8 pf = as_vec<V8>(u32x4{dsp[o4], dsp[o4 + 1], dsp[o4 + 2], dsp[o4 + 3]});
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Kt + ks * 16 * TL::ROWB + voff[db][0]));
                    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Kt + ks * 16 * TL::ROWB + voff[db][1]));
                    const u32x2 a0 = __builtin_bit_cast(u32x2, lo), a1 = __builtin_bit_cast(u32x2, hi4);
                    dqacc[db] = mfma32x32x16(as_vec<V8>(u32x4{a0[0], a0[1], a1[0], a1[1]}), pf, dqacc[db]);
                }
            }
        }
    };

    if (MASK & MASK_BLOCK) {
        BlockWalk walk(p.bm + b * p.bm_sb + h * p.bm_sh + (int64_t)qt * p.bm_sq, kt_hi);
        const int nkb = kt_hi;
        int cv, nv;
        int cur = walk.next(0, lane, cv);
        int nxt = cur < nkb ? walk.next(cur + 1, lane, nv) : nkb;
        if (cur < nkb) load_tile(cur, kv0, kv0 + TILEB);
        kv_barrier<0>();
        // one tile per iteration, the two buffers alternating (a second unrolled copy of
        // the tile body, as in the dense loop, pushes this variant past 256 VGPRs)
        int st = 0;
        while (cur < nkb) {
            unsigned char *Kc = st ? kv1 : kv0, *Kn = st ? kv0 : kv1;
            tile(cur, cv, Kc, Kc + TILEB, nxt < nkb ? nxt : -1, Kn, Kn + TILEB);
            kv_barrier<0>();
            cur = nxt;
            cv = nv;
            st ^= 1;
            if (cur < nkb) nxt = walk.next(cur + 1, lane, nv);
        }
    } else {
        if (kt_lo < kt_hi) load_tile(kt_lo, kv0, kv0 + TILEB);
        kv_barrier<0>();
        for (int kt = kt_lo; kt < kt_hi; kt += 2) {
            tile(kt, 1, kv0, kv0 + TILEB, kt + 1 < kt_hi ? kt + 1 : -1, kv1, kv1 + TILEB);
            kv_barrier<0>();
            if (kt + 1 < kt_hi) {
                tile(kt + 1, 1, kv1, kv1 + TILEB, kt + 2 < kt_hi ? kt + 2 : -1, kv0, kv0 + TILEB);
                kv_barrier<0>();
            }
        }
    }

    // dQ through LDS (every wave is past its last tile): each wave's own 32-row slice
    store_rows_via_lds<TT, D>(dqacc, p.scale, (wave_s < 4 ? kv0 : kv1) + (wave_s & 3) * 32 * TL::ROWB,
                              (uint16_t *)p.dq + b * p.dq_sb + h * p.dq_sh + (int64_t)r0 * p.dq_ss, p.dq_ss,
                              p.Sq - r0, lane);
}

// ---- dK, dV: one workgroup = NW waves x 32 keys of one (b, kv head) ----
// (one wave per SIMD: K^T, V^T and the dK, dV accumulators of a wave's 32 keys take
// most of a 512-register budget, the dK/dV accumulators living in AGPRs; 64-row query
// tiles give four independent MFMA chains for S and dP)
template <typename TT, int D, bool ALIBI, int MASK, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(BwdParams p) {
    constexpr int BQ = 64;          // query rows per tile
    constexpr int RB = BQ / 32;     // 32-row blocks per tile
    constexpr int BNK = 32 * NW;    // keys per workgroup
    constexpr int KS = D / 16, DB = D / 32;
    typedef Tile<D> TL;
    constexpr int TILEB = BQ * TL::ROWB;       // bytes of one Q (or dO) tile
    constexpr int LOADS = TILEB / 1024 / NW;   // copies per wave per tensor per tile
    constexpr int RPI = 1024 / TL::ROWB;
    typedef typename TT::vec8 V8;
    static_assert(LOADS >= 1 && LOADS * NW * 1024 == TILEB, "tile shape");
    static_assert(kBwdRowPad % BQ == 0, "workspace row padding");

    // per stage: Q tile, dO tile, then the tile rows' lse2 and -D (64 floats each), and
    // with the document mask their 64 query document ids (read from LDS by the tile: a
    // global load inside it would make the compiler wait for the copy in flight)
    constexpr int STAGEB = 2 * TILEB + 2 * BQ * 4 + ((MASK & MASK_DOC) ? BQ * 4 : 0);
    __shared__ __attribute__((aligned(1024))) unsigned char qd0[STAGEB];
    __shared__ __attribute__((aligned(1024))) unsigned char qd1[STAGEB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    // causal: the first key tiles are seen by the most queries; they start first
    int kt, pair;
    work_item(blockIdx.x, gridDim.x, p.n_tiles, (MASK & MASK_CAUSAL) != 0, kt, pair);
    if (MASK & MASK_CAUSAL) kt = p.n_tiles - 1 - kt;
    const int hk = pair % p.Hkv;
    const int b = pair / p.Hkv;
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int kw0 = kt * BNK + wave_s * 32;  // this wave's first key
    const int key = kw0 + l32;               // the key this lane owns
    const bool key_ok = key < p.Skv;

    // K^T and V^T fragments (B operands): key `key`, dims 16*ks + 8*hi .. +7
    V8 kf[KS], vf[KS];
    {
        const int kk = key_ok ? key : 0;
        const uint16_t *kr = (const uint16_t *)p.k + b * p.k_sb + hk * p.k_sh + (int64_t)kk * p.k_ss + 8 * hi;
        const uint16_t *vr = (const uint16_t *)p.v + b * p.v_sb + hk * p.v_sh + (int64_t)kk * p.v_ss + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = as_vec<V8>(key_ok ? *(const u32x4 *)(kr + 16 * ks) : u32x4{0, 0, 0, 0});
            vf[ks] = as_vec<V8>(key_ok ? *(const u32x4 *)(vr + 16 * ks) : u32x4{0, 0, 0, 0});
        }
    }

    // query rows that can see this workgroup's keys
    const int kmin = kt * BNK, kmax = min(kt * BNK + BNK, p.Skv) - 1;
    int i_lo = 0, i_hi = p.Sq;
    if ((MASK & MASK_CAUSAL) && !(MASK & MASK_BLOCK)) i_lo = kmin;
    if ((MASK & MASK_WINDOW) && !(MASK & MASK_BLOCK)) {
        i_hi = min(i_hi, kmax + p.window + 1);
        if (!(MASK & MASK_CAUSAL)) i_lo = max(0, kmin - p.window);
    }
    // packed documents: rows of the documents of the tile's keys; per wave, the document
    // ids of its first and last keys and, per lane, of its key
    int wk_lo = 0, wk_hi = 0, mykdoc = 0;
    if ((MASK & MASK_DOC) && p.Skv > 0) {
        const int32_t *qd = p.qdoc + b * p.qdoc_sb, *kd = p.kvdoc + b * p.kvdoc_sb;
        if (!(MASK & MASK_BLOCK)) {
            int dlo, dhi;
            wave_search_range(qd, p.Sq, kd[kmin], kd[kmax], lane, dlo, dhi);
            i_lo = max(i_lo, dlo);
            i_hi = min(i_hi, dhi);
        }
        wk_lo = kd[min(kw0, p.Skv - 1)];
        wk_hi = kd[min(kw0 + 31, p.Skv - 1)];
        mykdoc = kd[min(key, p.Skv - 1)];
    }
    const int qt_lo = i_lo / BQ;
    const int qt_hi = i_hi > i_lo ? (i_hi + BQ - 1) / BQ : qt_lo;
    const int nq = qt_hi - qt_lo;
    const int n_it = p.group * nq;  // (query head of the group, q tile) pairs

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
    uint32_t qgo[LOADS], dgo[LOADS];
    int trow[LOADS], tchunk[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        const int r = (wave_s * LOADS + i) * RPI + lane / TL::CH;
        const int c = (lane % TL::CH) ^ TL::swz(r);
        trow[i] = r;
        tchunk[i] = c;
        qgo[i] = (uint32_t)(r * (int)p.q_ss + 8 * c) * 2u;
        dgo[i] = (uint32_t)(r * (int)p.do_ss + 8 * c) * 2u;
    }
    // copy the Q and dO rows of iteration n (query head h, tile qt)
    auto load_tile = [&](int n, unsigned char *dst) {
        const int h = hk * p.group + n / nq, i0 = (qt_lo + n % nq) * BQ;
        const uint16_t *qg = (const uint16_t *)p.q + b * p.q_sb + h * p.q_sh;
        const uint16_t *dg = (const uint16_t *)p.dout + b * p.do_sb + h * p.do_sh;
        const uint32_t ql = lds_addr(dst) + (uint32_t)(wave_s * LOADS) * 1024u;
        const uint32_t dl = ql + TILEB;
        if (wave_s == 0) {
            // the rows' lse2 and -D (the (b, h) row block is padded to whole tiles)
            const int64_t w = ((int64_t)b * p.Hq + h) * p.sq_pad + i0 + lane;
            const uint32_t sl = lds_addr(dst) + 2 * TILEB;
            dma4_vaddr(p.ws_lse2 + w, sl);
            dma4_vaddr(p.ws_nd + w, sl + BQ * 4);
            // the rows' document ids, clamped to the last row
            if (MASK & MASK_DOC) dma4_vaddr(p.qdoc + b * p.qdoc_sb + min(i0 + lane, p.Sq - 1), sl + 2 * BQ * 4);
        }
        if (i0 + BQ <= p.Sq) {
            const char *qb = (const char *)(qg + (int64_t)i0 * p.q_ss);
            const char *db_ = (const char *)(dg + (int64_t)i0 * p.do_ss);
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                dma16_sbase(qb, qgo[i], ql + i * 1024);
                dma16_sbase(db_, dgo[i], dl + i * 1024);
            }
        } else {
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int gr = min(i0 + trow[i], p.Sq - 1);
                dma16_vaddr(qg + (int64_t)gr * p.q_ss + 8 * tchunk[i], ql + i * 1024);
                dma16_vaddr(dg + (int64_t)gr * p.do_ss + 8 * tchunk[i], dl + i * 1024);
            }
        }
    };

    f32x16 dkacc[DB], dvacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        dkacc[db] = f32x16{};
        dvacc[db] = f32x16{};
    }

    auto tile = [&](int n, const unsigned char *Qt, int next, unsigned char *Nn) {
        if (next >= 0) load_tile(next, Nn);
        const unsigned char *Dt = Qt + TILEB;
        const int h = hk * p.group + n / nq, i0 = (qt_lo + n % nq) * BQ;
        const int i_last = i0 + BQ - 1;
        int blk = 1;
        if ((MASK & MASK_BLOCK) && kw0 < p.Skv)
            blk = p.bm[b * p.bm_sb + h * p.bm_sh + (int64_t)(i0 / kBlockQ) * p.bm_sq + kw0 / kBlockKV];
        const bool pred = blk == 1;
        bool skip = blk == 0 || kw0 >= p.Skv;
        bool need_mask = kw0 + 31 >= p.Skv || i_last >= p.Sq;
        if ((MASK & MASK_CAUSAL) && pred) {
            skip |= i_last < kw0;
            need_mask |= i0 < kw0 + 31;
        }
        if ((MASK & MASK_WINDOW) && pred) {
            skip |= (kw0 - i_last > p.window) || (i0 - (kw0 + 31) > p.window);
            need_mask |= max(i_last - kw0, kw0 + 31 - i0) > p.window;
        }
        bool doc_mask = false;
        const int32_t *qd = (const int32_t *)(Qt + 2 * TILEB + 2 * BQ * 4);  // the rows' ids, clamped
        if ((MASK & MASK_DOC) && pred && !skip) {
            const int qdl = qd[0], qdh = qd[BQ - 1];
            skip |= qdh < wk_lo || qdl > wk_hi;
            doc_mask = !(wk_lo == wk_hi && qdl == qdh && qdl == wk_lo);
            need_mask |= doc_mask;
        }
        if (skip) return;
        // a tile that straddles documents: the rows of the lane's key's document,
        // [dfirst, dend) as offsets in the 64-row tile
        int dfirst = 0, dend = BQ;
        if ((MASK & MASK_DOC) && doc_mask) tile_doc_range(qd[lane], mykdoc, dfirst, dend);
        // per-lane rows of block rb of the accumulator: i0 + 32*rb + 8*a + 4*hi + (0..3),
        // their lse2 and -D from the copy in LDS (pad rows hold no data and are masked)
        const float *sl2 = (const float *)(Qt + 2 * TILEB), *snd = sl2 + BQ;
        f32x4 l2[RB][4];
        // S = Q K^T and dP - D = dO V^T - D (a lane: one key, 16 rows per 32-row block;
        // the dP accumulators start at the rows' -D)
        f32x16 sacc[RB], dpacc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            sacc[rb] = f32x16{};
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                l2[rb][a] = *(const f32x4 *)(sl2 + 32 * rb + 8 * a + 4 * hi);
                const f32x4 nd = *(const f32x4 *)(snd + 32 * rb + 8 * a + 4 * hi);
#pragma unroll
                for (int c = 0; c < 4; ++c) dpacc[rb][4 * a + c] = nd[c];
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const u32x4 qa = *(const u32x4 *)(Qt + rb * 32 * TL::ROWB + koff[ks]);
                const u32x4 da = *(const u32x4 *)(Dt + rb * 32 * TL::ROWB + koff[ks]);
                sacc[rb] = mfma32x32x16(as_vec<V8>(qa), kf[ks], sacc[rb]);
                dpacc[rb] = mfma32x32x16(as_vec<V8>(da), vf[ks], dpacc[rb]);
            }
        // operand reads two k-steps ahead of their MFMAs (with one wave per SIMD
        // nothing else hides an LDS latency); the first group also takes the rows'
        // lse2 and D reads above (8 per 32-row block)
        __builtin_amdgcn_sched_group_barrier(0x100, 8 * RB + 4 * RB, 0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * RB, 0);
            if (ks + 2 < KS) __builtin_amdgcn_sched_group_barrier(0x100, 2 * RB, 0);
        }
        float slope2 = 0.f;
        if (ALIBI) slope2 = (p.slopes ? p.slopes[h] : exp2f(-8.f * (float)(h + 1) / (float)p.Hq)) * kLog2e;
        uint32_t pp[RB][8], dsp[RB][8];
        // general: scale and alibi applied to the score; masked: the predicates too
        auto make = [&](bool general, bool masked) {
            // the lane's kept rows in this tile: one interval of offsets io = i - i0 -
            // 4*hi (each predicate keeps an interval; a key past Skv keeps none)
            int ilo = 0, ihi = 0;
            if (masked) {
                const int relk = key - i0 - 4 * hi;
                ihi = key_ok ? p.Sq - i0 - 4 * hi : 0;
                if ((MASK & MASK_CAUSAL) && pred) ilo = max(ilo, relk);
                if ((MASK & MASK_WINDOW) && pred) {
                    ilo = max(ilo, relk - p.window);
                    ihi = min(ihi, relk + p.window + 1);
                }
                if ((MASK & MASK_DOC) && pred) {
                    ilo = max(ilo, dfirst - 4 * hi);
                    ihi = min(ihi, dend - 4 * hi);
                }
            }
            const uint32_t span = ihi > ilo ? (uint32_t)(ihi - ilo) : 0u;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    float pv[2], ds[2];
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        const int e = 2 * e2 + u;
                        const float lse2 = l2[rb][e >> 2][e & 3];
                        float x;
                        if (general) {
                            const int io = 32 * rb + 8 * (e >> 2) + (e & 3);
                            const int i = i0 + 4 * hi + io;
                            const float t = ALIBI ? fmaf(sacc[rb][e], c2, slope2 * (float)(key - i)) : sacc[rb][e] * c2;
                            const bool keep = !masked || (uint32_t)(io - ilo) < span;
                            x = keep ? fast_exp2(t - lse2) : 0.f;
                            ds[u] = keep ? x * dpacc[rb][e] : 0.f;
                        } else {
                            x = fast_exp2(fmaf(sacc[rb][e], c2, -lse2));
                            ds[u] = x * dpacc[rb][e];
                        }
                        pv[u] = x;
                    }
                    pp[rb][e2] = pack2(pv[0], pv[1], TT{});
                    dsp[rb][e2] = pack2(ds[0], ds[1], TT{});
                }
        };
        if (need_mask)
            make(true, true);
        else if (ALIBI)
            make(true, false);
        else
            make(false, false);
        // dV += P^T dO and dK += dS^T Q over the tile's 16-row k-steps
#pragma unroll
        for (int ks = 0; ks < BQ / 16; ++ks) {
            const int rb = ks >> 1, o4 = 4 * (ks & 1);
            const V8 pa = as_vec<V8>(u32x4{pp[rb][o4], pp[rb][o4 + 1], pp[rb][o4 + 2], pp[rb][o4 + 3]});
            const V8 sa = as_vec<V8>(u32x4{dsp[rb][o4], dsp[rb][o4 + 1], dsp[rb][o4 + 2], dsp[rb][o4 + 3]});
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const s16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Dt + ks * 16 * TL::ROWB + voff[db][0]));
                const s16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Dt + ks * 16 * TL::ROWB + voff[db][1]));
                const s16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Qt + ks * 16 * TL::ROWB + voff[db][0]));
                const s16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Qt + ks * 16 * TL::ROWB + voff[db][1]));
                const u32x2 d0 = __builtin_bit_cast(u32x2, dlo), d1 = __builtin_bit_cast(u32x2, dhi);
                const u32x2 q0 = __builtin_bit_cast(u32x2, qlo), q1 = __builtin_bit_cast(u32x2, qhi);
                dvacc[db] = mfma32x32x16(pa, as_vec<V8>(u32x4{d0[0], d0[1], d1[0], d1[1]}), dvacc[db]);
                dkacc[db] = mfma32x32x16(sa, as_vec<V8>(u32x4{q0[0], q0[1], q1[0], q1[1]}), dkacc[db]);
            }
        }
        // the transposed reads of a 16-row step issued one step ahead of its MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4 * DB, 1);
#pragma unroll
        for (int ks = 0; ks < BQ / 16; ++ks) {
            if (ks + 1 < BQ / 16) __builtin_amdgcn_sched_group_barrier(0x100, 4 * DB, 1);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * DB, 1);
        }
    };

    if constexpr ((MASK & MASK_BLOCK) && BNK == kBlockKV) {
        // The workgroup's keys are one block column of the block mask, so an item's
        // class is the same for all its waves: items whose block is empty are skipped
        // outright (no copy, no barrier). Their classes are read 64 items at a time, a
        // byte per lane, and walked by ballot; every wave derives the same sequence.
        int wbase = -64, wv = 0;
        uint64_t wm = 0;
        auto next_item = [&](int from) -> int {
            while (from < n_it) {
                if (from >= wbase + 64) {
                    wbase = from & ~63;
                    const int t = wbase + lane;
                    wv = 0;
                    if (t < n_it) {
                        const int h = hk * p.group + t / nq, qt = qt_lo + t % nq;
                        wv = p.bm[b * p.bm_sb + h * p.bm_sh + (int64_t)(qt * BQ / kBlockQ) * p.bm_sq + kt];
                    }
                    wm = __builtin_amdgcn_ballot_w64(wv != 0);
                }
                const uint64_t m = wm & (~0ull << (from - wbase));
                if (m) return wbase + (int)__builtin_ctzll(m);
                from = wbase + 64;
            }
            return n_it;
        };
        int cur = next_item(0);
        if (cur < n_it) load_tile(cur, qd0);
        kv_barrier<0>();
        while (cur < n_it) {
            const int nx = next_item(cur + 1);
            tile(cur, qd0, nx < n_it ? nx : -1, qd1);
            kv_barrier<0>();
            if (nx >= n_it) break;
            cur = next_item(nx + 1);
            tile(nx, qd1, cur < n_it ? cur : -1, qd0);
            kv_barrier<0>();
        }
    } else {
        if (n_it > 0) load_tile(0, qd0);
        kv_barrier<0>();
        for (int n = 0; n < n_it; n += 2) {
            tile(n, qd0, n + 1 < n_it ? n + 1 : -1, qd1);
            kv_barrier<0>();
            if (n + 1 < n_it) {
                tile(n + 1, qd1, n + 2 < n_it ? n + 2 : -1, qd0);
                kv_barrier<0>();
            }
        }
    }

    // accumulator layout: lane holds dim 32*db + l32, keys kw0 + 8*(e/4) + 4*hi + e%4.
    // dK, then dV, go through the wave's own 32-key slice of LDS (every wave is past its
    // last tile) in the Q tile layout and leave as whole rows, 16 bytes per lane, instead
    // of 2 bytes per lane and store
    unsigned char *os = qd0 + wave_s * 32 * TL::ROWB;
    constexpr int RPS = 64 / TL::CH;  // rows per store instruction
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const f32x16 *acc = t == 0 ? dkacc : dvacc;
        const float mul = t == 0 ? p.scale : 1.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int kk = 8 * (e >> 2) + 4 * hi + (e & 3), d = 32 * db + l32;
                *(uint16_t *)(os + TL::off(kk, d >> 3) + 2 * (d & 7)) = narrow1(acc[db][e] * mul, TT{});
            }
        uint16_t *g = t == 0 ? (uint16_t *)p.dk + b * p.dk_sb + hk * p.dk_sh + (int64_t)kw0 * p.dk_ss
                             : (uint16_t *)p.dv + b * p.dv_sb + hk * p.dv_sh + (int64_t)kw0 * p.dv_ss;
        const int64_t ss = t == 0 ? p.dk_ss : p.dv_ss;
#pragma unroll
        for (int i = 0; i < 32 / RPS; ++i) {
            const int rr = i * RPS + lane / TL::CH, c = lane % TL::CH;
            const u32x4 y = *(const u32x4 *)(os + TL::off(rr, c));
            if (kw0 + rr < p.Skv) *(u32x4 *)(g + (int64_t)rr * ss + 8 * c) = y;
        }
    }
}

template <typename TT, int D, bool A, int M>
hipError_t launch_bwd_one(BwdParams p, hipStream_t s) {
    // dK/dV workgroup: 4 waves (128 keys); with a block mask 2 waves, so that its 64
    // keys are one block column and empty blocks skip whole items
    constexpr int NW = (M & MASK_BLOCK) ? 2 : 4;
    // dQ workgroup: 8 waves (256 rows share each K/V tile) without a mask or with
    // causal alone, as in the forward (each 1-1.5% faster overall at S = 8192); other
    // masks keep 128-row tiles
    constexpr int NWQ = (M == 0 || M == MASK_CAUSAL) ? 8 : 4;
    const int64_t nrows = (int64_t)p.B * p.Hq * p.Sq;
    if (nrows > 0) {
        const int rpb = 256 / (D / 8);
        bwd_pre_kernel<TT, D><<<dim3((unsigned)((nrows + rpb - 1) / rpb)), dim3(256), 0, s>>>(p);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        BwdParams q = p;
        q.n_tiles = (p.Sq + 32 * NWQ - 1) / (32 * NWQ);
        bwd_dq_kernel<TT, D, A, M, NWQ><<<dim3((unsigned)(q.n_tiles * p.Hq * p.B)), dim3(64 * NWQ), 0, s>>>(q);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if ((int64_t)p.B * p.Hkv * p.Skv > 0) {
        BwdParams k = p;
        k.n_tiles = (p.Skv + 32 * NW - 1) / (32 * NW);
        bwd_dkdv_kernel<TT, D, A, M, NW><<<dim3((unsigned)(k.n_tiles * p.Hkv * p.B)), dim3(64 * NW), 0, s>>>(k);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename TT, int D>
hipError_t launch_bwd_t(const BwdParams &p, bool alibi, int mask, hipStream_t s) {
#define MM_CASE(A, M) case (A) * 16 + (M): return launch_bwd_one<TT, D, (A) != 0, (M)>(p, s);
    switch ((alibi ? 16 : 0) + (mask & 15)) {
        MM_CASE(0, 0) MM_CASE(0, 1) MM_CASE(0, 2) MM_CASE(0, 3)
        MM_CASE(0, 4) MM_CASE(0, 5) MM_CASE(0, 6) MM_CASE(0, 7)
        MM_CASE(0, 8) MM_CASE(0, 9) MM_CASE(0, 10) MM_CASE(0, 11)
        MM_CASE(0, 12) MM_CASE(0, 13) MM_CASE(0, 14) MM_CASE(0, 15)
        MM_CASE(1, 0) MM_CASE(1, 1) MM_CASE(1, 2) MM_CASE(1, 3)
        MM_CASE(1, 4) MM_CASE(1, 5) MM_CASE(1, 6) MM_CASE(1, 7)
        MM_CASE(1, 8) MM_CASE(1, 9) MM_CASE(1, 10) MM_CASE(1, 11)
        MM_CASE(1, 12) MM_CASE(1, 13) MM_CASE(1, 14) MM_CASE(1, 15)
        default: return hipErrorInvalidValue;
    }
#undef MM_CASE
}

}  // namespace mm
