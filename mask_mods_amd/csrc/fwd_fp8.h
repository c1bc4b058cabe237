// fwd_fp8.h -- flash-attention forward for gfx950 on fp8 (OCP e4m3) inputs, bf16 output.
//
// Same flex semantics and tiling as the 16-bit kernel (fwd_mfma.h): a wave owns 32 query
// rows, keys stream through LDS in 64-key tiles copied by DMA, both products run in
// transposed form on the MFMA with fp32 accumulation. Here the MFMA is the gfx950
// 32x32x64 f8f6f4 instruction with e4m3 operands on both sides:
//   S^T[j][i] = sum_d K8[j][d] Q8[i][d]    A = K tile (2 x ds_read_b128 per 64 dims),
//                                          B = Q8^T held in VGPRs
//   O^T[d][i] += sum_j V8^T[d][j] P8^T[j][i]
// with the per-tensor dequantisation factors applied outside the products: the Q and
// K factors multiply the score scale, the V factor the output.
//
// P is rounded to e4m3 (round to nearest even) to feed the second product. The lane's
// 32 scores of a tile (S^T accumulator elements of two 32-key blocks) are exactly the
// 32 contraction slots it holds in the B operand, taken in accumulator order, so P never
// moves between lanes. V^T comes from the row-major V tile through ds_read_b64_tr_b8:
// in each 16-lane group, output lane t receives byte t%8 of the 8 bytes addressed by
// input lanes 2k + t/8 (k = 0..7); pairs of input lanes read the same key at dims
// 8 apart, so lane t gets one dim over 8 keys, and four reads give the 32 keys of the
// lane's slots. The row sum l is taken by one more MFMA with an all-ones A operand
// on the same rounded P, so O = sum(P8 V) / sum(P8) is normalised consistently.
//
// LDS: K and V tiles as 64 rows of D bytes; 16-byte chunks XOR-swizzled by row so the
// K reads (16 consecutive rows, one chunk) and the transposed V reads (8 keys x 2 chunks
// per 16 lanes) are free of bank conflicts.
#pragma once

#include "fwd_common.h"
#include "fwd_tile.h"

namespace mm {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
    // formats 0/0 = e4m3 for A and B; no block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// two e4m3 values (round to nearest even) into the low or high half of a word
// (the low-half write keeps the high half of `a`'s register, which pack_fp8_hi replaces)
__device__ __forceinline__ int pack_fp8_lo(float a, float b) {
    return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
}
__device__ __forceinline__ int pack_fp8_hi(float a, float b, int w) { return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, true); }

// Swizzled row-major tile of D one-byte elements per key.
template <int D>
struct Tile8 {
    static constexpr int ROWB = D;       // bytes per key row
    static constexpr int CH = D / 16;    // 16-byte chunks per row
    __host__ __device__ static constexpr int swz(int r) {
        // D = 128: j = (r >> 1) & 7 with its two low bits swapped; D = 64: (r >> 2) & 3
        return D == 128 ? (((r >> 1) & 1) << 1 | ((r >> 2) & 1) | ((r >> 1) & 4)) : ((r >> 2) & 3);
    }
    __host__ __device__ static constexpr int off(int r, int c) { return r * ROWB + 16 * (c ^ swz(r)); }
};

template <int D, bool ALIBI, int MASK, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_fp8_kernel(FwdParams p) {
    constexpr int BM = 32 * NW, BN = 64;
    constexpr int NC = D / 64;   // 64-dim k-steps of Q K^T
    constexpr int DB = D / 32;   // 32-dim blocks of O^T
    constexpr int NKB = BN / 32; // 32-key blocks of S^T per tile
    typedef Tile8<D> TL;
    constexpr int TILEB = BN * TL::ROWB;   // bytes of one K (or V) tile
    constexpr int KBLK = TILEB / 1024;     // 1 KB copy blocks per K tile
    constexpr int NL = 2 * KBLK / NW;      // copy instructions per wave per tile
    constexpr int RPI = 1024 / TL::ROWB;   // rows per copy block
    constexpr float kRescale = 8.f;
    static_assert(NL >= 1 && NL * NW == 2 * KBLK && KBLK % NL == 0, "tile shape");

    // no score_mod and no mask: the fixed-max fast path (see the end of the kernel)
    constexpr bool FAST = MASK == 0 && !ALIBI;
    __shared__ int wg_failed;

    // three stages, each a K tile then a V tile, then with the document mask the tile's 64
    // key document ids (read from LDS: a global load in a tile would make the compiler wait
    // for every copy in flight, the next tile's included)
    constexpr int DOCB = (MASK & MASK_DOC) ? 1024 : 0;
    __shared__ __attribute__((aligned(1024))) unsigned char kv0[2 * TILEB + DOCB];
    __shared__ __attribute__((aligned(1024))) unsigned char kv1[2 * TILEB + DOCB];
    __shared__ __attribute__((aligned(1024))) unsigned char kv2[2 * TILEB + DOCB];
    // the epilogue stages each wave's 32 rows of bf16 O (TILEB bytes) through LDS, two
    // waves per stage; 8-wave workgroups need a fourth region (one workgroup per CU)
    __shared__ __attribute__((aligned(1024))) unsigned char kv3[NW > 6 ? 2 * TILEB : 16];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // causal without a window: the last query tiles carry the most keys; they start first
    int qt, pair;
    work_item(blockIdx.x, gridDim.x, p.n_qtiles, longest_first(MASK), qt, pair);
    const int h = pair % p.Hq;
    const int b = pair / p.Hq;
    const int q0 = qt * BM;
    const int hk = h / p.group;

    const uint8_t *qg = (const uint8_t *)p.q + b * p.q_sb + h * p.q_sh;
    const uint8_t *kg = (const uint8_t *)p.k + b * p.k_sb + hk * p.k_sh;
    const uint8_t *vg = (const uint8_t *)p.v + b * p.v_sb + hk * p.v_sh;

    // the wave index as a scalar: tile classifications derived from it are wave-uniform
    // branches, not per-lane masked code
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int r0 = q0 + wave_s * 32;  // first row of this wave
    const int row = r0 + l32;

    // Q^T fragments (B operand): row `row`, dims 64*c + 32*hi .. +31. 4-wave workgroups
    // copy their 128 rows (clamped to the last row) by DMA into stage kv2, whole rows per
    // instruction, as two 64-row tiles in the K tile layout; the copy is in flight during
    // the document search and the first K/V copies, and the waves read their fragments
    // after the first barrier (the pass's first body refills kv2 only after a second one)
    constexpr bool QLDS = NW == 4;
    i32x8 qf[NC];
    if (QLDS) {
        constexpr int KB8 = (64 * Tile8<D>::ROWB) / 1024, NQ = 2 * KB8 / NW, RPB = 1024 / Tile8<D>::ROWB;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            const int blk = wave_s * NQ + i, t2 = blk / KB8;
            const int r = (blk % KB8) * RPB + lane / Tile8<D>::CH;
            const int gr = min(q0 + 64 * t2 + r, p.Sq - 1);
            dma16_vaddr(qg + (int64_t)gr * p.q_ss + 16 * ((lane % Tile8<D>::CH) ^ Tile8<D>::swz(r)),
                        lds_addr(kv2) + (uint32_t)(blk * 1024));
        }
    } else {
        const bool ok = row < p.Sq;
        const uint8_t *qr = qg + (int64_t)(ok ? row : 0) * p.q_ss + 32 * hi;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4 x0 = ok ? *(const u32x4 *)(qr + 64 * c) : u32x4{0, 0, 0, 0};
            const u32x4 x1 = ok ? *(const u32x4 *)(qr + 64 * c + 16) : u32x4{0, 0, 0, 0};
            qf[c] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
        }
    }

    const int row_max = min(q0 + BM, p.Sq) - 1;
    int j_lo = 0, j_hi = p.Skv;
    if ((MASK & MASK_CAUSAL) && !(MASK & MASK_BLOCK)) j_hi = min(j_hi, row_max + 1);
    if ((MASK & MASK_WINDOW) && !(MASK & MASK_BLOCK)) {
        j_lo = max(0, q0 - p.window);
        if (!(MASK & MASK_CAUSAL)) j_hi = min(j_hi, row_max + p.window + 1);
    }
    if (MASK & MASK_DOC) {
        // packed documents: only keys whose document lies within the tile's rows' range
        const int32_t *qd = p.qdoc + b * p.qdoc_sb, *kd = p.kvdoc + b * p.kvdoc_sb;
        if (!(MASK & MASK_BLOCK)) {
            int dlo, dhi;
            wave_search_range(kd, p.Skv, qd[q0], qd[row_max], lane, dlo, dhi);
            j_lo = max(j_lo, dlo);
            j_hi = min(j_hi, dhi);
        }
    }
    // document ids of the wave's first and last rows and of the lane's row
    int wd_lo = 0, wd_hi = 0, mydoc = 0;
    if (MASK & MASK_DOC) {
        const int32_t *qd = p.qdoc + b * p.qdoc_sb;
        wd_lo = qd[min(r0, p.Sq - 1)];
        wd_hi = qd[min(r0 + 31, p.Sq - 1)];
        mydoc = qd[min(row, p.Sq - 1)];
    }
    const int kt_lo = j_lo / BN;
    const int kt_hi = j_hi > j_lo ? (j_hi + BN - 1) / BN : kt_lo;

    float slope2 = 0.f;
    if (ALIBI) slope2 = (p.slopes ? p.slopes[h] : exp2f(-8.f * (float)(h + 1) / (float)p.Hq)) * kLog2e;
    const float c2 = p.scale_log2;

    // K reads: row l32 (+32 per key block), chunks 4c + 2hi + {0, 1}
    int koff[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        koff[c][0] = TL::off(l32, 4 * c + 2 * hi);
        koff[c][1] = TL::off(l32, 4 * c + 2 * hi + 1);
    }
    // transposed V reads: group G = lane/16, u = lane%16 addresses key
    // 8*(u/8) + 4*(G/2) + (u/2)%4 (+16 per read), dims 32*db + 16*(G%2) + 8*(u%2)
    int voff[DB];
    {
        const int G = lane >> 4, u = lane & 15;
        const int key = 8 * (u >> 3) + 4 * (G >> 1) + ((u >> 1) & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) voff[db] = TL::off(key, 2 * db + (G & 1)) + 8 * (u & 1);
    }

    // copies: wave w moves blocks w*NL .. +NL-1 of the tile pair (K blocks first, then V)
    const bool cp_v = wave_s * NL >= KBLK;
    const int blk0 = wave_s * NL - (cp_v ? KBLK : 0);
    const uint8_t *cp_src = cp_v ? vg : kg;
    const int64_t cp_ss = cp_v ? p.v_ss : p.k_ss;
    uint32_t goff[NL];
    int trow[NL], tchunk[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int r = (blk0 + i) * RPI + lane / TL::CH;
        const int c = (lane % TL::CH) ^ TL::swz(r);
        trow[i] = r;
        tchunk[i] = c;
        goff[i] = (uint32_t)(r * (int)cp_ss + 16 * c);
    }
    auto load_tile = [&](int kt, unsigned char *kdst) {
        const int k0 = kt * BN;
        const uint32_t dst = lds_addr(kdst) + (cp_v ? (uint32_t)TILEB : 0u) + (uint32_t)blk0 * 1024u;
        if ((MASK & MASK_DOC) && wave_s == 0)
            dma4_vaddr(p.kvdoc + b * p.kvdoc_sb + min(k0 + lane, p.Skv - 1), lds_addr(kdst) + 2 * TILEB);
        if (k0 + BN <= p.Skv) {
            const uint8_t *base = cp_src + (int64_t)k0 * cp_ss;
#pragma unroll
            for (int i = 0; i < NL; ++i) dma16_sbase(base, goff[i], dst + i * 1024);
        } else {
#pragma unroll
            for (int i = 0; i < NL; ++i) {
                const int gr = min(k0 + trow[i], p.Skv - 1);
                dma16_vaddr(cp_src + (int64_t)gr * cp_ss + 16 * tchunk[i], dst + i * 1024);
            }
        }
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    f32x16 lacc = f32x16{};
    float m_run = -INFINITY;
    const int one4 = 0x38383838;  // four e4m3 ones
    const i32x8 ones = {one4, one4, one4, one4, one4, one4, one4, one4};

    // ---- the four phases of a tile ----
    // S^T of the tile in stage Kt (raw dot products)
    auto qk = [&](const unsigned char *Kt, f32x16 (&sacc)[NKB]) {
        u32x4 ka[NKB][NC][2];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int e = 0; e < 2; ++e) ka[kb][c][e] = *(const u32x4 *)(Kt + kb * 32 * TL::ROWB + koff[c][e]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const u32x4 x0 = ka[kb][c][0], x1 = ka[kb][c][1];
                const i32x8 a = {(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                 (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                sacc[kb] = mfma_fp8(a, qf[c], sacc[kb]);
            }
        }
    };
    // scale / score_mod / mask_mod where the tile needs them; returns the multiplier the
    // exponent (and the max) apply to sacc: 1 when sacc was rewritten as base-2 scores,
    // else the scale (plain tiles keep the raw dot products)
    auto transform = [&](int kt, int blk, const unsigned char *St, f32x16 (&sacc)[NKB]) -> float {
        const int k0 = kt * BN;
        const int r_last = r0 + 31;
        const bool pred = blk == 1;
        bool dead = false, need_mask = k0 + BN > p.Skv;
        if ((MASK & MASK_CAUSAL) && pred) {
            dead |= k0 > r_last;
            need_mask |= k0 + BN - 1 > r0;
        }
        if ((MASK & MASK_WINDOW) && pred) {
            dead |= (k0 - r_last > p.window) || (r0 - (k0 + BN - 1) > p.window);
            need_mask |= max(r_last - k0, k0 + BN - 1 - r0) > p.window;
        }
        bool doc_mask = false;
        const int32_t *kd = (const int32_t *)(St + 2 * TILEB);  // the tile's key ids, clamped
        if ((MASK & MASK_DOC) && pred) {
            const int kdl = kd[0], kdh = kd[BN - 1];
            dead |= kdh < wd_lo || kdl > wd_hi;
            doc_mask = !dead && !(wd_lo == wd_hi && kdl == kdh && kdl == wd_lo);
            need_mask |= !(wd_lo == wd_hi && kdl == kdh && kdl == wd_lo);
        }
        if (!(ALIBI || need_mask || !(c2 > 0.f))) return c2;
        const float base = ALIBI ? slope2 * (float)(k0 + 4 * hi - row) : 0.f;
        // a tile that straddles documents: the lane's document's keys, [dfirst, dend)
        int dfirst = 0, dend = BN;
        if ((MASK & MASK_DOC) && doc_mask) tile_doc_range(kd[lane], mydoc, dfirst, dend);
        // the lane's kept keys in the tile: one interval of offsets jo = j - k0 - 4*hi
        // (each predicate keeps an interval; a dead tile keeps none)
        const int rel = row - k0 - 4 * hi;
        int jlo = 0, jhi = dead ? 0 : p.Skv - k0 - 4 * hi;
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
        auto scores = [&](bool masked) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int jo = 32 * kb + 8 * (e >> 2) + (e & 3);
                    float t = ALIBI ? fmaf(sacc[kb][e], c2, fmaf(slope2, (float)jo, base)) : sacc[kb][e] * c2;
                    if (masked) t = (uint32_t)(jo - jlo) < span ? t : -INFINITY;
                    sacc[kb][e] = t;
                }
            }
        };
        // one uniform branch, then straight-line code for the whole tile
        if (need_mask) scores(true);
        else scores(false);
        return 1.f;
    };
    // the tile's row max (in base-2 units) over both lane halves
    auto tile_max = [&](const f32x16 (&sacc)[NKB], float cc) -> float {
        float m = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, sacc[kb][e]);
        return m * cc;
    };
    // lazy rescale: raise the running max only when the tile exceeds it by > 2^8
    auto rescale = [&](float mloc) {
        mloc = row_max2(mloc);
        if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescale)) {
            const float m_new = fmaxf(m_run, mloc);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            lacc *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
    };
    // P = 2^(t - m) rounded to e4m3; byte i of the operand is accumulator element i % 16
    // of key block i / 16
    auto expcvt = [&](const f32x16 (&sacc)[NKB], float cc, int (&pp)[8]) {
        const float nm = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int kb = w >> 2, e0 = 4 * (w & 3);
            const float x0 = fast_exp2(fmaf(sacc[kb][e0 + 0], cc, nm));
            const float x1 = fast_exp2(fmaf(sacc[kb][e0 + 1], cc, nm));
            const float x2 = fast_exp2(fmaf(sacc[kb][e0 + 2], cc, nm));
            const float x3 = fast_exp2(fmaf(sacc[kb][e0 + 3], cc, nm));
            pp[w] = pack_fp8_hi(x2, x3, pack_fp8_lo(x0, x1));
        }
    };
    // O^T += V^T P^T (the row sum, ones x P, is issued with the products of S)
    auto pv = [&](const unsigned char *Vt, const int (&pp)[8]) {
        const i32x8 pf = {pp[0], pp[1], pp[2], pp[3], pp[4], pp[5], pp[6], pp[7]};
        i32x2 va[DB][4];
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                va[db][r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((MM_LDS i32x2 *)(Vt + voff[db] + 16 * r * TL::ROWB));
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const i32x8 a = {va[db][0][0], va[db][0][1], va[db][1][0], va[db][1][1],
                             va[db][2][0], va[db][2][1], va[db][3][0], va[db][3][1]};
            oacc[db] = mfma_fp8(a, pf, oacc[db]);
        }
    };

    // ---- software pipeline over the visited tiles t_0, t_1, ... ----
    // Iteration n copies t_{n+2} into the free stage, computes S of t_{n+1} on the MFMA
    // while the VALU turns S of t_n into P, then runs P V of t_n while the VALU scales,
    // masks and reduces S of t_{n+1}. Three LDS stages hold t_n (its V), t_{n+1} (its K)
    // and the copy in flight. The MFMAs of t_{n+1} are issued even past the last tile
    // (on stale data, results unused) so the iteration stays one straight-line block.
    constexpr int END = 1 << 30;
    BlockWalk walk((MASK & MASK_BLOCK) ? p.bm + b * p.bm_sb + h * p.bm_sh + (int64_t)qt * p.bm_sq : nullptr,
                   kt_hi);
    auto next_tile = [&](int t, int &cls) -> int {
        if (t >= END) { cls = 0; return END; }
        if (MASK & MASK_BLOCK) {
            const int n = walk.next(t + 1, lane, cls);
            return n < kt_hi ? n : END;
        }
        cls = 1;
        return t + 1 < kt_hi ? t + 1 : END;
    };
    // One pass over the row's tiles. fast: the row's max is fixed by its first tile and
    // later tiles neither take their max nor rescale (no score_mod, unmasked only; see
    // below); otherwise the lazy rescale. compute: this wave computes; a wave that does
    // not only copies its share of each tile and meets the barriers.
    auto run = [&](bool fast, bool compute) __attribute__((always_inline)) {
        int c_cur, c_nxt, c_aft;
        int cur;
        if (MASK & MASK_BLOCK) {
            cur = walk.next(0, lane, c_cur);
            if (cur >= kt_hi) cur = END;
        } else {
            cur = kt_lo < kt_hi ? kt_lo : END;
            c_cur = 1;
        }
        if (cur >= END) return;
        int nxt = next_tile(cur, c_nxt);
        int aft = next_tile(nxt, c_aft);
        load_tile(cur, kv0);
        load_tile(nxt < END ? nxt : cur, kv1);
        kv_barrier<0>();
        f32x16 s_cur[NKB];
        float cc_cur = 1.f;
        if (compute) {
            qk(kv0, s_cur);
            cc_cur = transform(cur, c_cur, kv0, s_cur);
            rescale(tile_max(s_cur, cc_cur));
        }
        auto body = [&](unsigned char *Sc, unsigned char *Sn, unsigned char *Sa) __attribute__((always_inline)) {
            load_tile(aft < END ? aft : cur, Sa);
            f32x16 s_nxt[NKB];
            float cc_nxt = 1.f;
            if (compute) {
                qk(Sn, s_nxt);
                int pp[8];
                expcvt(s_cur, cc_cur, pp);
                lacc = mfma_fp8(ones, i32x8{pp[0], pp[1], pp[2], pp[3], pp[4], pp[5], pp[6], pp[7]}, lacc);
                // interleave: the K reads first, then each MFMA of S(t_{n+1}) followed by
                // a share of the exponentials of t_n
                __builtin_amdgcn_sched_group_barrier(0x100, NKB * NC * 2, 0);
#pragma unroll
                for (int i = 0; i < NKB * NC; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                cc_nxt = transform(nxt < END ? nxt : cur, c_nxt, Sn, s_nxt);
                pv(Sc + TILEB, pp);
                if (!fast) {
                    const float mloc = tile_max(s_nxt, cc_nxt);
                    // then the V reads, and each MFMA of P V followed by a share of the max
                    __builtin_amdgcn_sched_group_barrier(0x100, 4 * DB, 0);
#pragma unroll
                    for (int i = 0; i < DB + 1; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                    }
                    // a tile past the end must not move the running max
                    rescale(nxt < END ? mloc : -INFINITY);
                }
            }
            kv_barrier<0>();
            if (compute) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) s_cur[kb] = s_nxt[kb];
                cc_cur = cc_nxt;
            }
        };
        auto advance = [&]() __attribute__((always_inline)) {
            cur = nxt;
            c_cur = c_nxt;
            nxt = aft;
            c_nxt = c_aft;
            aft = next_tile(aft, c_aft);
        };
        for (;;) {
            body(kv0, kv1, kv2);
            if (nxt >= END) break;
            advance();
            body(kv1, kv2, kv0);
            if (nxt >= END) break;
            advance();
            body(kv2, kv0, kv1);
            if (nxt >= END) break;
            advance();
        }
    };

    if constexpr (FAST) {
        // Without a score_mod or mask the row's max is fixed by its first tile, and later
        // tiles exponentiate against it without taking their own max (32 maxima, a
        // cross-lane exchange and the rescale test per wave-tile). A P above e4m3's range
        // (a score more than about 8.9, base 2, above that max) converts to NaN, which the
        // all-ones product carries into the row sum; a row whose sum is not finite marks
        // its wave, and the workgroup then streams the tiles once more: the failed waves
        // recompute from scratch with the lazy rescale (every P at most 2^8), the others
        // only copy.
        if (tid == 0) wg_failed = 0;
        run(true, true);
        const bool wave_failed = __builtin_amdgcn_ballot_w64(!(lacc[0] <= 3.0e38f)) != 0;
        if (wave_failed && lane == 0) wg_failed = 1;
        __syncthreads();
        if (wg_failed) {
            if (wave_failed) {
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
                lacc = f32x16{};
                m_run = -INFINITY;
            }
            run(false, wave_failed);
        }
    } else {
        // every other case: one pass with the lazy rescale (the loop above written out
        // once more, so that these kernels compile exactly as before the fast path)
        int c_cur, c_nxt, c_aft;
        int cur;
        if (MASK & MASK_BLOCK) {
            cur = walk.next(0, lane, c_cur);
            if (cur >= kt_hi) cur = END;
        } else {
            cur = kt_lo < kt_hi ? kt_lo : END;
            c_cur = 1;
        }
        if (cur < END) {
            int nxt = next_tile(cur, c_nxt);
            int aft = next_tile(nxt, c_aft);
            load_tile(cur, kv0);
            load_tile(nxt < END ? nxt : cur, kv1);
            kv_barrier<0>();
            if (QLDS) {
                const unsigned char *qs = kv2 + wave_s * 32 * TL::ROWB;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const u32x4 x0 = *(const u32x4 *)(qs + koff[c][0]), x1 = *(const u32x4 *)(qs + koff[c][1]);
                    qf[c] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                                  (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
                }
                kv_barrier<0>();
            }
            f32x16 s_cur[NKB];
            qk(kv0, s_cur);
            float cc_cur = transform(cur, c_cur, kv0, s_cur);
            rescale(tile_max(s_cur, cc_cur));
            auto body = [&](unsigned char *Sc, unsigned char *Sn, unsigned char *Sa) {
                load_tile(aft < END ? aft : cur, Sa);
                f32x16 s_nxt[NKB];
                qk(Sn, s_nxt);
                int pp[8];
                expcvt(s_cur, cc_cur, pp);
                lacc = mfma_fp8(ones, i32x8{pp[0], pp[1], pp[2], pp[3], pp[4], pp[5], pp[6], pp[7]}, lacc);
                // interleave: the K reads first, then each MFMA of S(t_{n+1}) followed by a
                // share of the exponentials of t_n
                __builtin_amdgcn_sched_group_barrier(0x100, NKB * NC * 2, 0);
    #pragma unroll
                for (int i = 0; i < NKB * NC; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                const float cc_nxt = transform(nxt < END ? nxt : cur, c_nxt, Sn, s_nxt);
                pv(Sc + TILEB, pp);
                const float mloc = tile_max(s_nxt, cc_nxt);
                // then the V reads, and each MFMA of P V followed by a share of the max
                __builtin_amdgcn_sched_group_barrier(0x100, 4 * DB, 0);
    #pragma unroll
                for (int i = 0; i < DB + 1; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
                }
                // a tile past the end must not move the running max
                rescale(nxt < END ? mloc : -INFINITY);
                kv_barrier<0>();
    #pragma unroll
                for (int kb = 0; kb < NKB; ++kb) s_cur[kb] = s_nxt[kb];
                cc_cur = cc_nxt;
            };
            auto advance = [&]() {
                cur = nxt;
                c_cur = c_nxt;
                nxt = aft;
                c_nxt = c_aft;
                aft = next_tile(aft, c_aft);
            };
            for (;;) {
                body(kv0, kv1, kv2);
                if (nxt >= END) break;
                advance();
                body(kv1, kv2, kv0);
                if (nxt >= END) break;
                advance();
                body(kv2, kv0, kv1);
                if (nxt >= END) break;
                advance();
            }
        }

    }

    // ---- epilogue: both lane halves hold the whole row sum in lacc ----
    const float l_tot = lacc[0];
    bool dropped = false;
    if (p.rowdrop) {
        const uint32_t rid = (uint32_t)(((int64_t)b * p.Hq + h) * p.Sq + row);
        dropped = fmix32(p.rd_seed ^ rid) < p.rd_thr;
    }
    const bool live = l_tot > 0.f && !dropped;
    const float inv = live ? p.v_descale / l_tot : 0.f;
    // O through LDS as whole rows, each wave in its own TILEB-byte slice, once every wave
    // is past its last tile (the wait also covers the Q copy of a workgroup with no tile)
    kv_barrier<0>();
    unsigned char *const os = wave_s < 2 ? kv0 : wave_s < 4 ? kv1 : wave_s < 6 ? kv2 : kv3;
    store_rows_via_lds<BF16, D>(oacc, inv, os + (wave_s & 1) * TILEB,
                                (uint16_t *)p.o + b * p.o_sb + h * p.o_sh + (int64_t)r0 * p.o_ss, p.o_ss,
                                p.Sq - r0, lane);
    if (row < p.Sq && hi == 0 && p.lse)
        p.lse[((int64_t)b * p.Hq + h) * p.Sq + row] = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, bool A, int M>
hipError_t launch_fwd_fp8_one(FwdParams p, hipStream_t s) {
    constexpr int NW = M == 0 ? 8 : 4;  // (8 waves for causal: 7% slower)
    p.n_qtiles = (p.Sq + 32 * NW - 1) / (32 * NW);
    const dim3 grid((unsigned)(p.n_qtiles * p.Hq * p.B)), block(64 * NW);
    fwd_fp8_kernel<D, A, M, NW><<<grid, block, 0, s>>>(p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_fp8(const FwdParams &p, bool alibi, int mask, hipStream_t s) {
#define MM_CASE(A, M) case (A) * 16 + (M): return launch_fwd_fp8_one<D, (A) != 0, (M)>(p, s);
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
