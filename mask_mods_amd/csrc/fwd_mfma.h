// fwd_mfma.h -- flash-attention forward for gfx950 with flex mods (bf16 / f16 inputs).
//
// One workgroup = NW waves = 32*NW query rows of one (batch, query head); each wave owns
// 32 rows. The default is 8 waves (256 rows, one workgroup per CU, two waves per SIMD):
// every K/V tile copied into LDS then serves 256 rows, which halves the L2 -> LDS
// traffic of a 4-wave layout. Keys/values stream through LDS in tiles of 64 keys in a
// two-stage ring: the next tile is copied global -> LDS by the DMA path
// (global_load_lds_dwordx4, no VGPR staging) while the current tile is computed.
//
// Both products run on the 32x32x16 MFMA with fp32 accumulation, in transposed form
// so that a lane always owns one query row:
//   S^T[j][i] = sum_d K[j][d] Q[i][d]      A = K tile (ds_read_b128), B = Q^T in VGPRs
//   O^T[d][i] += sum_j V^T[d][j] P^T[j][i] A = V^T read with ds_read_b64_tr_b16 from the
//                                          row-major V tile, B = P^T from registers
// In the C layout a lane holds column i = lane % 32 and 16 rows, so the softmax
// reductions over keys are lane-local plus one exchange with lane ^ 32, and the
// per-row rescale of O is a per-lane scalar multiply. The contraction index of
// V^T P^T (the key) is consumed in the order the S^T accumulator hands keys to each
// lane, so P^T needs no data movement.
//
// K and V tiles are stored row-major (one key per row) with the 16-byte chunks of each
// row XOR-swizzled by the row index, which keeps both the K reads (32 rows, one chunk)
// and the transposed V reads (4 rows, two chunks per 16 lanes) free of bank conflicts.
//
// Softmax: scores are kept in base-2 units (t = scale*log2(e)*q.k [+ slope*log2(e)*(j-i)]).
// The running max is only raised when a tile's max exceeds it by more than 2^8 in
// probability (lazy rescale): P then stays <= 256, exact in the final O / l. Tiles with
// no mask or score_mod skip the max altogether: they exponentiate against the running
// max and fall back to the max only if a lane's sum of P exceeds 256. Row sums add the
// fp32 P values; the PV product takes them rounded to 16 bits.
// Semantics (FlyDSL PR #931, Summary): score_mod sees the scaled score, the mask_mod is
// applied after it, and rows with no kept key give O = 0, LSE = -inf (the running max
// is clamped to 0 while it is -inf, and the epilogue guards 1/l).
#pragma once

#include "fwd_common.h"
#include "fwd_pipe.h"
#include "fwd_tile.h"

namespace mm {

template <typename TT, int D, bool ALIBI, int MASK, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_mfma_kernel(FwdParams p) {
    constexpr int BM = 32 * NW, BN = 64;
    constexpr int KS = D / 16;    // k-steps of Q K^T
    constexpr int DB = D / 32;    // 32-row blocks of O^T
    constexpr int NKB = BN / 32;  // 32-key blocks of S^T per tile
    typedef Tile<D> TL;
    constexpr int TILEB = BN * TL::ROWB;            // bytes of one K (or V) tile
    constexpr int LOADS = TILEB / 1024 / NW;        // DMA instructions per wave per tile
    constexpr int RPI = 1024 / TL::ROWB;            // rows per DMA instruction
    constexpr float kRescale = 8.f;                 // lazy-rescale threshold (log2 units)
    constexpr float kRescaleSum = 256.f;            // 2^kRescale: bound on a plain tile's lane sum
    typedef typename TT::vec8 V8;
    static_assert(LOADS >= 1 && LOADS * NW * 1024 == TILEB, "tile shape");

    // The two K/V buffers as distinct LDS objects: the loop below is unrolled by two so
    // every tile reads a statically known buffer while the DMA fills the other, and the
    // compiler can see the reads never alias the in-flight copies (no early vmcnt wait).
    // (one object per stage, K then V: the waitcnt pass tracks only a few DMA targets)
    // with the document mask a stage also holds its tile's 64 key document ids (copied
    // with K and V), so that a tile reads them from LDS: a global load inside the tile
    // would make the compiler wait for every copy in flight, the next tile's included
    constexpr int DOCB = (MASK & MASK_DOC) ? 1024 : 0;
    __shared__ __attribute__((aligned(1024))) unsigned char kv0[2 * TILEB + DOCB];
    __shared__ __attribute__((aligned(1024))) unsigned char kv1[2 * TILEB + DOCB];
    unsigned char *const KB[2] = {kv0, kv1};
    unsigned char *const VB[2] = {kv0 + TILEB, kv1 + TILEB};

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // causal without a window: the last query tiles carry the most keys; they start first
    int qt, pair;
    work_item(blockIdx.x, gridDim.x, p.n_qtiles, longest_first(MASK), qt, pair);
    const int h = pair % p.Hq;
    const int b = pair / p.Hq;
    const int q0 = qt * BM;
    const int hk = h / p.group;

    const uint16_t *qg = (const uint16_t *)p.q + b * p.q_sb + h * p.q_sh;
    const uint16_t *kg = (const uint16_t *)p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vg = (const uint16_t *)p.v + b * p.v_sb + hk * p.v_sh;

    // the wave index as a scalar: tile classifications derived from it are wave-uniform
    // branches, not per-lane masked code
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const int r0 = q0 + wave_s * 32;  // first row of this wave
    const int row = r0 + l32;       // the row this lane owns

    // Q^T fragments (B operand): row `row`, dims 16*ks + 8*hi .. +7
    // 4-wave workgroups copy their 128 Q rows to LDS instead: whole rows per copy
    // instruction rather than 32 bytes of 32 rows per lane load. Rows q0 .. q0+127
    // (clamped to the last row) become two 64-row tiles in stage 1, in the K tile layout;
    // the copy is issued first, so that it is in flight during the key-range search and
    // the first K/V copy. Each wave reads its rows' fragments as the K fragments are
    // read (q_read below), and a barrier then frees stage 1 for the loop.
    constexpr bool QLDS = NW == 4;
    V8 qf[KS];
    if (QLDS) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
            for (int i = 0; i < LOADS; ++i) {
                const int r = (wave_s * LOADS + i) * RPI + lane / TL::CH;
                const int gr = min(q0 + 64 * t2 + r, p.Sq - 1);
                dma16_vaddr(qg + (int64_t)gr * p.q_ss + 8 * ((lane % TL::CH) ^ TL::swz(r)),
                            lds_addr(kv1) + (uint32_t)(t2 * TILEB + (wave_s * LOADS + i) * 1024));
            }
    } else {
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
    // with a block mask, full blocks bypass the predicates: no analytic key range
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

    // ---- per-lane LDS offsets (bytes, within one tile) ----
    // K (A operand of S^T): row 32*kb + l32, chunk 2*ks + hi
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = TL::off(l32, 2 * ks + hi);
    // V^T via transpose reads: lane = 16*G + t reads row 16*ks + 8*m2 + 4*hi + t/4,
    // dims 32*db + 16*(G%2) + 4*(t%4) .. +3; the 16 lanes then hold V[rows][d] transposed.
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

    // ---- DMA of one K and one V tile ----
    // Each wave copies LOADS blocks of 1 KB per tile; block `blk` holds tile rows
    // blk*RPI .. +RPI-1 and lane L lands in LDS slot L of the block: tile row
    // r = blk*RPI + L/CH, chunk slot L%CH, which receives global chunk (L%CH) ^ swz(r).
    // The lane's byte offset inside a tile is loop-invariant (32-bit; the host bounds
    // 64*stride); full tiles add a wave-uniform base so the copy uses the
    // scalar-base + vector-offset address form. The tile that crosses Skv clamps rows
    // to the last key instead (their scores are masked).
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

    auto q_read = [&]() {
        const unsigned char *qs = kv1 + wave_s * 32 * TL::ROWB;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const V8 *)(qs + koff[ks]);
    };

    f32x16 oacc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;

    // ---- the pieces of one tile ----
    // Whether this wave skips tile kt, and whether the tile needs per-pair masking.
    // `blk` is the tile's block-mask class: 1 = the mask_mod predicates decide,
    // 2 = every pair kept (predicates not evaluated).
    auto classify = [&](int kt, int blk, const unsigned char *Kt, bool &need_mask, bool &doc_mask) -> bool {
        const int k0 = kt * BN;
        const int r_last = r0 + 31;
        const bool pred = blk == 1;  // predicates apply in this tile
        bool skip = kt >= kt_hi;
        need_mask = k0 + BN > p.Skv;
        doc_mask = false;
        if ((MASK & MASK_CAUSAL) && pred) {
            skip |= k0 > r_last;
            need_mask |= k0 + BN - 1 > r0;
        }
        if ((MASK & MASK_WINDOW) && pred) {
            skip |= (k0 - r_last > p.window) || (r0 - (k0 + BN - 1) > p.window);
            need_mask |= max(r_last - k0, k0 + BN - 1 - r0) > p.window;
        }
        if ((MASK & MASK_DOC) && pred && !skip) {
            const int32_t *kd = (const int32_t *)(Kt + 2 * TILEB);  // the tile's ids, clamped
            const int kdl = kd[0], kdh = kd[BN - 1];
            skip |= kdh < wd_lo || kdl > wd_hi;
            doc_mask = !(wd_lo == wd_hi && kdl == kdh && kdl == wd_lo);
            need_mask |= doc_mask;
        }
        return skip;
    };
    // S^T = K Q^T for the tile in Kt
    auto qk = [&](const unsigned char *Kt, f32x16 (&sacc)[NKB]) {
        if (MASK & MASK_BLOCK) {
            // the block walk holds a few more registers: fragments of one 32-key block
            // at a time keep the loop within 256 VGPRs
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                u32x4 ka[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) ka[ks] = *(const u32x4 *)(Kt + kb * 32 * TL::ROWB + koff[ks]);
                sacc[kb] = f32x16{};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) sacc[kb] = mfma32x32x16(as_vec<V8>(ka[ks]), qf[ks], sacc[kb]);
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // DS reads of block kb
                __builtin_amdgcn_sched_group_barrier(0x008, KS, 0);  // its MFMAs
            }
            return;
        }
        // all K fragments first, then the MFMAs: the reads overlap each other instead of
        // each MFMA waiting on its own read
        u32x4 ka[NKB][KS];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) ka[kb][ks] = *(const u32x4 *)(Kt + kb * 32 * TL::ROWB + koff[ks]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            sacc[kb] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) sacc[kb] = mfma32x32x16(as_vec<V8>(ka[kb][ks]), qf[ks], sacc[kb]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, NKB * KS, 0);  // DS reads
        __builtin_amdgcn_sched_group_barrier(0x008, NKB * KS, 0);  // then MFMAs
    };
    // scale, score_mod and mask_mod, the running max (lazily rescaling O and l), then
    // P = 2^(t - m) as 16-bit pairs and the row sum
    // tdoc: with doc_mask, the document id of key k0 + lane (clamped to the last key)
    auto softmax = [&](int kt, int blk, bool need_mask, bool doc_mask, int tdoc, f32x16 (&sacc)[NKB],
                       uint32_t (&pp)[NKB][8]) {
        const int k0 = kt * BN;
        const bool pred = blk == 1;
        // scores in base-2 units; lane's keys: k0 + 32*kb + 8*(e/4) + 4*hi + e%4.
        // general tiles (alibi, masking, non-positive scale) store t in sacc and use
        // cc = 1; plain tiles keep the raw dot products and fold the scale into the
        // exponent (cc = scale*log2e > 0 commutes with the max).
        float mloc = -INFINITY, cc;
        const bool general = ALIBI || need_mask || !(c2 > 0.f);
        if (general) {
            const float base = ALIBI ? slope2 * (float)(k0 + 4 * hi - row) : 0.f;
            // the lane's document's keys in this tile, [dfirst, dend) as tile offsets
            int dfirst = 0, dend = BN;
            if ((MASK & MASK_DOC) && doc_mask) tile_doc_range(tdoc, mydoc, dfirst, dend);
            // with alibi, one copy with the predicates and one without, chosen per tile:
            // inlined separately, so the unmasked copy (alibi tiles off the diagonal)
            // carries no per-score compare and select. Without alibi a general tile
            // nearly always needs the predicates (and they keep every pair of a tile
            // that does not), so only the masked copy is emitted.
            // Every predicate keeps an interval of keys (j < Skv; causal j <= row; window
            // |row - j| <= w; the document's keys [dfirst, dend)), so the lane's kept keys
            // in this tile are one interval of the offsets jo = j - k0 - 4*hi: [jlo, jlo +
            // span). Each score then costs one subtraction and one unsigned compare. The
            // host keeps Sq, Skv < 2^30 and the window <= max(Sq, Skv), so no bound overflows.
            const int rel = row - k0 - 4 * hi;  // the row as an offset jo
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
            auto scores = [&](bool masked) __attribute__((always_inline)) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int jo = 32 * kb + 8 * (e >> 2) + (e & 3);
                        float t = ALIBI ? fmaf(sacc[kb][e], c2, fmaf(slope2, (float)jo, base)) : sacc[kb][e] * c2;
                        if (masked) t = (uint32_t)(jo - jlo) < span ? t : -INFINITY;
                        sacc[kb][e] = t;
                        mloc = fmaxf(mloc, t);
                    }
                }
            };
            if (ALIBI && !need_mask)
                scores(false);
            else
                scores(true);
            cc = 1.f;
        } else {
            // plain tile: exponentiate against the running max as it stands. Each P is
            // non-negative, so a lane sum of at most 2^8 bounds every P by 2^8, the bound
            // the max test below keeps; the tile takes the max (and maybe the rescale)
            // only when some lane's sum is larger or not finite (no max yet: m = -inf
            // gives +inf exponents).
            float psum = 0.f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e2 = 0; e2 < 8; ++e2) {
                    const float x0 = fast_exp2(fmaf(sacc[kb][2 * e2], c2, -m_run));
                    const float x1 = fast_exp2(fmaf(sacc[kb][2 * e2 + 1], c2, -m_run));
                    pp[kb][e2] = pack2(x0, x1, TT{});
                    psum += x0;
                    psum += x1;
                }
            if (!__builtin_amdgcn_ballot_w64(!(psum <= kRescaleSum))) {
                l_run += psum;
                return;
            }
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, sacc[kb][e]);
            mloc *= c2;
            cc = c2;
        }
        mloc = row_max2(mloc);
        // lazy rescale: raise the running max only when the tile exceeds it by > 2^8
        if (__builtin_amdgcn_ballot_w64(mloc > m_run + kRescale)) {
            const float m_new = fmaxf(m_run, mloc);
            const float alpha = fast_exp2(m_run - (m_new == -INFINITY ? 0.f : m_new));
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
        const float nm = m_run == -INFINITY ? 0.f : -m_run;
        // P = 2^(t - m) as 16-bit pairs for the PV product; the row sum adds the fp32
        // values (a sum of the 16-bit roundings would put up to 2^-9 of relative
        // error into the LSE of rows with few keys)
        float psum = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float x0 = fast_exp2(fmaf(sacc[kb][2 * e2], cc, nm));
                const float x1 = fast_exp2(fmaf(sacc[kb][2 * e2 + 1], cc, nm));
                pp[kb][e2] = pack2(x0, x1, TT{});
                psum += x0;
                psum += x1;
            }
        l_run += psum;
    };
    // O^T += V^T P^T for the tile in Vt (all transposed V reads first, then the MFMAs)
    auto pv = [&](const unsigned char *Vt, const uint32_t (&pp)[NKB][8]) {
        if (MASK & MASK_BLOCK) {
            // fragments of one 16-key step at a time (register pressure, as in qk)
#pragma unroll
            for (int ks = 0; ks < BN / 16; ++ks) {
                u32x4 va[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (MM_LDS s16x4 *)(Vt + ks * 16 * TL::ROWB + voff[db][0]));
                    const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (MM_LDS s16x4 *)(Vt + ks * 16 * TL::ROWB + voff[db][1]));
                    const u32x2 a0 = __builtin_bit_cast(u32x2, lo), a1 = __builtin_bit_cast(u32x2, hi4);
                    va[db] = u32x4{a0[0], a0[1], a1[0], a1[1]};
                }
                const int kb = ks >> 1, o4 = 4 * (ks & 1);
                const V8 pf = as_vec<V8>(u32x4{pp[kb][o4], pp[kb][o4 + 1], pp[kb][o4 + 2], pp[kb][o4 + 3]});
#pragma unroll
                for (int db = 0; db < DB; ++db) oacc[db] = mfma32x32x16(as_vec<V8>(va[db]), pf, oacc[db]);
            }
#pragma unroll
            for (int ks = 0; ks < BN / 16; ++ks) {
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * DB, 1);  // transposed V reads
                __builtin_amdgcn_sched_group_barrier(0x008, DB, 1);      // their MFMAs
            }
            return;
        }
        u32x4 va[BN / 16][DB];
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (MM_LDS s16x4 *)(Vt + ks * 16 * TL::ROWB + voff[db][0]));
                const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (MM_LDS s16x4 *)(Vt + ks * 16 * TL::ROWB + voff[db][1]));
                const u32x2 a0 = __builtin_bit_cast(u32x2, lo), a1 = __builtin_bit_cast(u32x2, hi4);
                va[ks][db] = u32x4{a0[0], a0[1], a1[0], a1[1]};
            }
#pragma unroll
        for (int ks = 0; ks < BN / 16; ++ks) {
            const int kb = ks >> 1, o4 = 4 * (ks & 1);
            const V8 pf = as_vec<V8>(u32x4{pp[kb][o4], pp[kb][o4 + 1], pp[kb][o4 + 2], pp[kb][o4 + 3]});
#pragma unroll
            for (int db = 0; db < DB; ++db) oacc[db] = mfma32x32x16(as_vec<V8>(va[ks][db]), pf, oacc[db]);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * (BN / 16) * DB, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, (BN / 16) * DB, 1);
    };

    // one tile, all phases in order: DMA tile `next` (if >= 0) into (Kn, Vn) while
    // computing tile kt on (Kt, Vt)
    auto tile = [&](int kt, int blk, const unsigned char *Kt, const unsigned char *Vt, int next,
                    unsigned char *Kn, unsigned char *Vn) {
        if (next >= 0) load_tile(next, Kn, Vn);
        bool need_mask, doc_mask;
        if (!classify(kt, blk, Kt, need_mask, doc_mask)) {
            // a tile that straddles documents: its 64 key ids, one per lane, from LDS
            int tdoc = 0;
            if ((MASK & MASK_DOC) && doc_mask) tdoc = ((const int32_t *)(Kt + 2 * TILEB))[lane];
            f32x16 sacc[NKB];
            qk(Kt, sacc);
            uint32_t pp[NKB][8];
            softmax(kt, blk, need_mask, doc_mask, tdoc, sacc, pp);
            pv(Vt, pp);
        }
    };

    if (MASK & MASK_BLOCK) {
        BlockWalk walk(p.bm + b * p.bm_sb + h * p.bm_sh + (int64_t)qt * p.bm_sq, kt_hi);
        const int nkb = kt_hi;  // key tiles (64 keys each) of the row
        auto next_block = [&](int from, int &val) { return walk.next(from, lane, val); };
        int cv, nv;
        int cur = next_block(0, cv);
        int nxt = cur < nkb ? next_block(cur + 1, nv) : nkb;
        if (cur < nkb) load_tile(cur, KB[0], VB[0]);
        kv_barrier<0>();
        if (QLDS) {
            q_read();
            kv_barrier<0>();
        }
        while (cur < nkb) {
            tile(cur, cv, KB[0], VB[0], nxt < nkb ? nxt : -1, KB[1], VB[1]);
            kv_barrier<0>();
            cur = nxt;
            cv = nv;
            if (cur >= nkb) break;
            nxt = next_block(cur + 1, nv);
            tile(cur, cv, KB[1], VB[1], nxt < nkb ? nxt : -1, KB[0], VB[0]);
            kv_barrier<0>();
            cur = nxt;
            cv = nv;
            if (cur < nkb) nxt = next_block(cur + 1, nv);
        }
    } else {
        if (kt_lo < kt_hi) load_tile(kt_lo, KB[0], VB[0]);
        kv_barrier<0>();
        if (QLDS) {
            q_read();
            kv_barrier<0>();
        }
        for (int kt = kt_lo; kt < kt_hi; kt += 2) {
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                if (kt + st < kt_hi) {
                    tile(kt + st, 1, KB[st], VB[st], kt + st + 1 < kt_hi ? kt + st + 1 : -1,
                         KB[st ^ 1], VB[st ^ 1]);
                    kv_barrier<0>();
                }
            }
        }
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
    // O through LDS (every wave is past its last tile): each wave's own 32-row slice
    store_rows_via_lds<TT, D>(oacc, inv, (wave_s < 4 ? kv0 : kv1) + (wave_s & 3) * 32 * TL::ROWB,
                              (uint16_t *)p.o + b * p.o_sb + h * p.o_sh + (int64_t)r0 * p.o_ss, p.o_ss,
                              p.Sq - r0, lane);
    if (row < p.Sq && hi == 0 && p.lse)
        p.lse[((int64_t)b * p.Hq + h) * p.Sq + row] = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
}


constexpr int kFwdNW = 8;          // waves per workgroup without a mask mod
constexpr int kFwdNWMasked = 4;    // window, document or block masks: finer row tiles skip more keys
constexpr int kFwdNWCausal = 8;    // causal alone on long rows: the shared tiles outweigh the idle diagonal waves
constexpr int kFwdCausalShort = 4096;  // causal without a score_mod, D = 128: at most this many visible keys -> 4 waves

template <typename TT, int D, bool A, int M, int NW>
hipError_t launch_fwd_mfma_nw(FwdParams p, hipStream_t s) {
    static_assert(!(M & MASK_BLOCK) || NW == 4, "block masks use 128-row workgroups");
    p.n_qtiles = (p.Sq + 32 * NW - 1) / (32 * NW);
    const dim3 grid((unsigned)(p.n_qtiles * p.Hq * p.B)), block(64 * NW);
    // the software-pipelined kernel: no score_mod, unmasked or causal, D = 128 with
    // 8-wave workgroups (its 96 KiB of LDS hold one per CU, two waves per SIMD). At D = 64
    // the halved MFMAs leave the same softmax work less to hide behind, and the
    // sequential kernel is faster.
    if constexpr (!A && (M == 0 || M == MASK_CAUSAL) && D == 128 && NW == 8)
        fwd_pipe_kernel<TT, D, M, NW><<<grid, block, 0, s>>>(p);
    else
        fwd_mfma_kernel<TT, D, A, M, NW><<<grid, block, 0, s>>>(p);
    return hipGetLastError();
}

template <typename TT, int D, bool A, int M>
hipError_t launch_fwd_mfma_one(FwdParams p, hipStream_t s) {
    // 8 waves (256 rows) share each K/V tile and halve the L2 -> LDS traffic. Causal
    // alone at D = 128 keeps 8 on long rows (at S = 8192 as fast as 4 without a
    // score_mod, 3% faster with alibi); without a score_mod it takes 4 when at most 4096
    // keys are visible (S 2048 and 4096: within 1% of the software-pipelined 8-wave
    // kernel), with alibi it keeps 8 there as well (3-9% faster than 4); with a window
    // or documents, 4-wave tiles (128 rows) follow the band
    // more closely and skip more key tiles, which matters more; a block mask's q-blocks
    // are 128 rows, one 4-wave workgroup each. D = 64 always takes 4: its halved tile
    // products leave the shared copies less to gain (no mod 7-15% faster at S 2048 to
    // 8192, causal 6-15%, alibi 0-3%)
    constexpr int NW = D == 64 ? 4 : (M == 0 ? kFwdNW : (M == MASK_CAUSAL ? kFwdNWCausal : kFwdNWMasked));
    if constexpr (M == MASK_CAUSAL && !A && NW != 4) {
        if ((p.Sq < p.Skv ? p.Sq : p.Skv) <= kFwdCausalShort) return launch_fwd_mfma_nw<TT, D, A, M, 4>(p, s);
    }
    return launch_fwd_mfma_nw<TT, D, A, M, NW>(p, s);
}

template <typename TT, int D>
hipError_t launch_fwd_mfma(const FwdParams &p, bool alibi, int mask, hipStream_t s) {
#define MM_CASE(A, M) case (A) * 16 + (M): return launch_fwd_mfma_one<TT, D, (A) != 0, (M)>(p, s);
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
