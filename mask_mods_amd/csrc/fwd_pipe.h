// fwd_pipe.h -- the 16-bit forward without a score_mod, unmasked or causal, as a
// software pipeline over 32-key blocks.
//
// Same tiling, data layout and numerics as fwd_mfma_kernel (a lane owns one query row,
// S^T = K Q^T and O^T += V^T P^T on the 32x32x16 MFMA, base-2 scores, fp32 row sums).
// What changes is the order of the work. In that kernel each tile runs QK, then the
// softmax, then PV, so a wave's VALU work and its MFMAs never overlap and the matrix
// pipe idles during every softmax. Here step u of a wave
//   - exponentiates the scores of key block u (VALU),
//   - computes S of block u+1 (QK MFMAs),
//   - accumulates P V of block u-1 (PV MFMAs),
// three independent streams, issued one MFMA at a time with a share of the exponentials
// and the LDS operand reads after each. A 32x32x16 MFMA occupies the matrix pipe for 32
// cycles and hides a few VALU instructions issued behind it; grouped instead, the same
// VALU work serialises with the MFMAs. Pipelining 32-key blocks rather than 64-key tiles
// keeps the extra state (one more S block and one more P block) within the 256
// registers of two waves per SIMD.
//
// The running max. The steady steps never rescale O: a conditional rescale of the O
// accumulators inside the loop makes the compiler keep a second copy of them and copy
// on every step. Instead each row's max is fixed by its first key block, and later
// blocks exponentiate against it, which is exact as long as no P exceeds 2^64 (2^15 for
// f16 P, below its largest finite value; fp32 O and l have ample headroom, and the
// 16-bit P keeps its relative precision). A block whose row sum of P leaves that bound
// (a score more than 64, or 15, above the first block's max in base 2) marks its wave
// failed. If any wave of the workgroup failed, the
// workgroup streams K and V twice more: the failed waves first take each row's exact
// max over all its keys (QK only), then recompute against it, where every P is at most
// 1 and nothing can fail. The other waves only do their share of the copies.
//
// LDS: K/V still arrive in 64-key tiles, one barrier per tile, two steps per tile.
// Tile iteration n runs steps 2n and 2n+1, which read K of tiles n and n+1 and V of
// tiles n-1 and n, while K of tile n+2 and V of tile n+1 are copied: three K slots and
// three V slots (96 KiB at D = 128), tile t in slot t mod 3. A wave needs a mask on its
// last block at most (the block crossing Skv, or its causal diagonal block), so the
// interleaved steps exponentiate unmasked blocks; a wave's first two iterations and its
// last ones take a sequential step that applies the mask where needed.
#pragma once

#include <type_traits>

#include "fwd_tile.h"

namespace mm {

template <typename TT, int D, int MASK, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_pipe_kernel(FwdParams p) {
    static_assert(MASK == 0 || MASK == MASK_CAUSAL, "the pipelined forward is unmasked or causal");
    constexpr bool CAUSAL = MASK == MASK_CAUSAL;
    constexpr int BM = 32 * NW, BN = 64, BK = 32;  // query rows, tile keys, block keys
    constexpr int KS = D / 16;             // k-steps of Q K^T = QK MFMAs per block
    constexpr int DB = D / 32;             // 32-row blocks of O^T
    constexpr int PPS = 8 / KS;            // pairs of scores exponentiated per MFMA pair
    constexpr int AHEAD = 2;               // operand reads issued this many MFMA pairs ahead
    typedef Tile<D> TL;
    constexpr int TILEB = BN * TL::ROWB;
    constexpr int LOADS = TILEB / 1024 / NW;
    constexpr int RPI = 1024 / TL::ROWB;
    // bound on a lane's sum of P in a block (so on every P): 2^64 for bf16 P, 2^15 for
    // f16 P, whose largest finite value is 65504
    constexpr float kFastSum = std::is_same<TT, F16>::value ? 32768.f : 18446744073709551616.f;
    typedef typename TT::vec8 V8;
    static_assert(LOADS >= 1 && LOADS * NW * 1024 == TILEB, "tile shape");
    static_assert((BK / 16) * DB == KS && PPS * KS == 8, "one QK and one PV MFMA per pair");

    // One array: K of tile t in slot t % 3 of the first half, its V in slot t % 3 of the
    // second. Every operand read is then a per-lane base register (K: the lane's offset
    // in a tile; V: the same plus the V half's start) plus an immediate below 64 KiB.
    __shared__ __attribute__((aligned(1024))) unsigned char smem[6 * TILEB];
    __shared__ int wg_failed;
    unsigned char *const k0s = smem, *const k1s = smem + TILEB, *const k2s = smem + 2 * TILEB;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // causal: the last query tiles carry the most keys; they start first
    int qt, pair;
    work_item(blockIdx.x, gridDim.x, p.n_qtiles, CAUSAL, qt, pair);
    const int h = pair % p.Hq;
    const int b = pair / p.Hq;
    const int q0 = qt * BM;
    const int hk = h / p.group;

    const uint16_t *qg = (const uint16_t *)p.q + b * p.q_sb + h * p.q_sh;
    const uint16_t *kg = (const uint16_t *)p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vg = (const uint16_t *)p.v + b * p.v_sb + hk * p.v_sh;

    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
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

    // key tiles of the workgroup; key blocks of the workgroup and of this wave (a wave
    // whose rows all lie past Sq computes nothing; with causal a wave stops at its
    // diagonal block, keys r0 .. r0 + 31)
    const int row_max = min(q0 + BM, p.Sq) - 1;
    const int j_hi = CAUSAL ? min(p.Skv, row_max + 1) : p.Skv;
    const int N = (j_hi + BN - 1) / BN;
    const int Nb = (j_hi + BK - 1) / BK;
    int Nbw = r0 < p.Sq ? Nb : 0;
    if (CAUSAL) Nbw = min(Nbw, r0 / BK + 1);
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
                voff[db][m2] = 3 * TILEB + TL::off(r, d >> 3) + 2 * (d & 7);
            }
    }

    // ---- DMA of one K or V tile: this wave's LOADS blocks of 1 KB (as fwd_mfma_kernel)
    int trow[LOADS], tchunk[LOADS];
    uint32_t kgo[LOADS], vgo[LOADS];  // the lane's byte offsets inside a full K / V tile
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
        trow[i] = (wave_s * LOADS + i) * RPI + lane / TL::CH;
        tchunk[i] = (lane % TL::CH) ^ TL::swz(trow[i]);
        kgo[i] = (uint32_t)(trow[i] * (int)p.k_ss + 8 * tchunk[i]) * 2u;
        vgo[i] = (uint32_t)(trow[i] * (int)p.v_ss + 8 * tchunk[i]) * 2u;
    }
    auto load_rows = [&](const uint16_t *g, int64_t ss, const uint32_t (&go)[LOADS], int kt,
                         unsigned char *dst) __attribute__((always_inline)) {
        const int k0 = kt * BN;
        const uint32_t l = lds_addr(dst) + (uint32_t)(wave_s * LOADS) * 1024u;
        if (k0 + BN <= p.Skv) {
            // the tile's base is wave-uniform; said explicitly so that it stays in SGPRs
            const uint64_t a = (uint64_t)(uintptr_t)(g + (int64_t)k0 * ss);
            // (readfirstlane returns int: both halves are zero-extended from uint32_t)
            const uint32_t ahi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
            const uint32_t alo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
            const char *base = (const char *)(uintptr_t)(((uint64_t)ahi << 32) | (uint64_t)alo);
            // a VALU write of an SGPR needs 5 wait states before a memory instruction reads
            // it, and the copies are inline asm the compiler does not look into
            asm volatile("s_nop 4" ::"s"(base));
#pragma unroll
            for (int i = 0; i < LOADS; ++i) dma16_sbase(base, go[i], l + i * 1024);
        } else {
            // the tile crossing Skv: rows past the end repeat the last key (masked)
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                dma16_vaddr(g + (int64_t)min(k0 + trow[i], p.Skv - 1) * ss + 8 * tchunk[i], l + i * 1024);
        }
    };
    // Tile iteration n copies K of tile n+2 into slot (n+2) % 3 and V of tile n+1 into
    // slot (n+1) % 3.
    auto copies = [&](int n, unsigned char *Kw, unsigned char *Vw) __attribute__((always_inline)) {
        if (n + 2 < N) load_rows(kg, p.k_ss, kgo, n + 2, Kw);
        if (n + 1 < N) load_rows(vg, p.v_ss, vgo, n + 1, Vw + 3 * TILEB);
    };

    // ---- operand fragments of one block (Kb / Vb: its first row in LDS) ----
    auto kfrag = [&](const unsigned char *Kb, int ks) __attribute__((always_inline)) -> u32x4 {
        return *(const u32x4 *)(Kb + koff[ks]);
    };
    // PV MFMA i of a block: 16-key step i / DB, 32-dim block i % DB
    auto vfrag = [&](const unsigned char *Vb, int i) __attribute__((always_inline)) -> u32x4 {
        const int kk = i / DB, db = i % DB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Vb + kk * 16 * TL::ROWB + voff[db][0]));
        const s16x4 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MM_LDS s16x4 *)(Vb + kk * 16 * TL::ROWB + voff[db][1]));
        const u32x2 a0 = __builtin_bit_cast(u32x2, lo), a1 = __builtin_bit_cast(u32x2, hi4);
        return u32x4{a0[0], a0[1], a1[0], a1[1]};
    };
    auto pfrag = [&](const uint32_t (&pp)[8], int i) __attribute__((always_inline)) -> V8 {
        const int o4 = 4 * (i / DB);
        return as_vec<V8>(u32x4{pp[o4], pp[o4 + 1], pp[o4 + 2], pp[o4 + 3]});
    };

    f32x16 oacc[DB];
    float m_run, l_run;
    bool failed;
    f32x16 s0, s1;          // S of block u in s0 / s1 by the parity of u
    uint32_t pb0[8], pb1[8];  // P of block u in pb0 / pb1 likewise

    // the block's base-2 score e, -inf where the mask drops the pair (block u's keys:
    // u*32 + 8*(e/4) + 4*hi + e%4)
    auto masked_t = [&](int u, const f32x16 &sacc, int e) __attribute__((always_inline)) -> float {
        const int j = u * BK + 8 * (e >> 2) + 4 * hi + (e & 3);
        bool keep = j < p.Skv;
        if (CAUSAL) keep &= j <= row;
        return keep ? sacc[e] * c2 : -INFINITY;
    };
    auto need_mask = [&](int u) __attribute__((always_inline)) -> bool {
        return u * BK + BK > p.Skv || (CAUSAL && u * BK + BK - 1 > r0);
    };
    // a block's P (masked as needed) against m_run, and its lane sum
    auto exp_block = [&](int u, const f32x16 &sacc, uint32_t (&pp)[8]) __attribute__((always_inline)) -> float {
        const float nm = m_run == -INFINITY ? 0.f : -m_run;
        float psum = 0.f;
        if (need_mask(u)) {
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float x0 = fast_exp2(masked_t(u, sacc, 2 * e2) + nm);
                const float x1 = fast_exp2(masked_t(u, sacc, 2 * e2 + 1) + nm);
                pp[e2] = pack2(x0, x1, TT{});
                psum += x0;
                psum += x1;
            }
        } else {
#pragma unroll
            for (int e2 = 0; e2 < 8; ++e2) {
                const float x0 = fast_exp2(fmaf(sacc[2 * e2], c2, nm));
                const float x1 = fast_exp2(fmaf(sacc[2 * e2 + 1], c2, nm));
                pp[e2] = pack2(x0, x1, TT{});
                psum += x0;
                psum += x1;
            }
        }
        return psum;
    };

    // Checks a block's lane sums against the bound (a failure marks the wave) and adds
    // them to l_run.
    auto settle = [&](float psum) __attribute__((always_inline)) {
        failed |= __builtin_amdgcn_ballot_w64(!(psum <= kFastSum)) != 0;
        l_run += psum;
    };

    // ---- sequential steps: a wave's first two iterations and its last ones ----
    auto qk_seq = [&](const unsigned char *Kb, f32x16 &sacc) __attribute__((always_inline)) {
        u32x4 ka[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ka[ks] = kfrag(Kb, ks);
        sacc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) sacc = mfma32x32x16(as_vec<V8>(ka[ks]), qf[ks], sacc);
    };
    auto pv_seq = [&](const unsigned char *Vb, const uint32_t (&pp)[8]) __attribute__((always_inline)) {
        u32x4 va[KS];
#pragma unroll
        for (int i = 0; i < KS; ++i) va[i] = vfrag(Vb, i);
#pragma unroll
        for (int i = 0; i < KS; ++i) oacc[i % DB] = mfma32x32x16(as_vec<V8>(va[i]), pfrag(pp, i), oacc[i % DB]);
    };
    // step u: QK of block u+1 (Kb), PV of block u-1 (Vb, pprev), the softmax of block u
    // (sc -> pcur); block 0 also sets the row's max (never lowering it)
    auto step_seq = [&](int u, const unsigned char *Kb, const unsigned char *Vb, f32x16 &sc, f32x16 &sn,
                        const uint32_t (&pprev)[8], uint32_t (&pcur)[8]) __attribute__((always_inline)) {
        if (u + 1 >= 0 && u + 1 < Nbw) qk_seq(Kb, sn);
        if (u >= 1 && u <= Nbw) pv_seq(Vb, pprev);
        if (u == 0 && Nbw > 0) {
            float mloc = -INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, masked_t(0, sc, e));
            m_run = fmaxf(m_run, row_max2(mloc));
            l_run += exp_block(0, sc, pcur);
        } else if (u >= 1 && u < Nbw) {
            settle(exp_block(u, sc, pcur));
        }
    };

    // ---- the interleaved step: softmax of the (unmasked) block in sc, S of the next
    // block into sn from Kb, P V of the previous block from Vb with pprev; P into pcur.
    // Chunk i runs QK MFMA i, the exponentials of score pair(s) i, PV MFMA i, the
    // packing and sums of pair(s) i - 1, and issues the operand reads AHEAD chunks on;
    // a scheduling barrier closes each chunk, so every chunk keeps exactly one MFMA of
    // each product with its share of the VALU work between them. The reads of the
    // step's first AHEAD chunks arrive in kpre / vpre (issued by the step before), and
    // its last chunks issue those of the next step (Kn / Vn) into the same registers, so
    // no step starts by waiting for the LDS.
    auto step_full = [&](const unsigned char *Kb, const unsigned char *Vb, const unsigned char *Kn,
                         const unsigned char *Vn, f32x16 &sc, f32x16 &sn, const uint32_t (&pprev)[8],
                         uint32_t (&pcur)[8], u32x4 (&kpre)[AHEAD], u32x4 (&vpre)[AHEAD]) __attribute__((always_inline)) {
        const float nm = -m_run;
        float ps0 = 0.f, ps1 = 0.f;
        u32x4 kf[KS], vf[KS];
        float x[8][2];
#pragma unroll
        for (int i = 0; i < AHEAD; ++i) {
            kf[i] = kpre[i];
            vf[i] = vpre[i];
        }
#pragma unroll
        for (int i = 0; i <= KS; ++i) {
            if (i < KS) {
                sn = mfma32x32x16(as_vec<V8>(kf[i]), qf[i], i == 0 ? f32x16{} : sn);
#pragma unroll
                for (int j = 0; j < PPS; ++j) {
                    const int e2 = i * PPS + j;
                    x[e2][0] = fast_exp2(fmaf(sc[2 * e2], c2, nm));
                    x[e2][1] = fast_exp2(fmaf(sc[2 * e2 + 1], c2, nm));
                }
                oacc[i % DB] = mfma32x32x16(as_vec<V8>(vf[i]), pfrag(pprev, i), oacc[i % DB]);
            }
            if (i > 0) {
#pragma unroll
                for (int j = 0; j < PPS; ++j) {
                    const int e2 = (i - 1) * PPS + j;
                    pcur[e2] = pack2(x[e2][0], x[e2][1], TT{});
                    asm volatile("" ::"v"(pcur[e2]));  // keeps the pack in its chunk
                    ps0 += x[e2][0];
                    ps1 += x[e2][1];
                }
            }
            if (i < KS) {
                const int r = i + AHEAD;  // the chunk whose operands are read now
                if (r < KS) {
                    kf[r] = kfrag(Kb, r);
                    vf[r] = vfrag(Vb, r);
                } else {
                    kpre[r - KS] = kfrag(Kn, r - KS);
                    vpre[r - KS] = vfrag(Vn, r - KS);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, PPS, 0);
                __builtin_amdgcn_sched_group_barrier(0x400, PPS, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, PPS, 0);
                __builtin_amdgcn_sched_group_barrier(0x400, PPS, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        settle(ps0 + ps1);
    };

    const int n_end = Nb >> 1;           // the tile iteration holding step Nb (the last PV)
    const int n_fast = (Nbw - 3) >> 1;   // iterations 1 .. n_fast run two interleaved steps
    // a sequential iteration, slots chosen at run time
    auto titer_seq = [&](int n) __attribute__((always_inline)) {
        const int r = (n + 3) % 3, r1 = r == 2 ? 0 : r + 1, r2 = r == 0 ? 2 : r - 1;
        unsigned char *const Kn = smem + r * TILEB, *const Kn1 = smem + r1 * TILEB, *const Vm = smem + r2 * TILEB;
        copies(n, Vm, Kn1);
        step_seq(2 * n, Kn + BK * TL::ROWB, Vm + BK * TL::ROWB, s0, s1, pb1, pb0);
        step_seq(2 * n + 1, Kn1, Kn, s1, s0, pb0, pb1);
        if (n < n_end) kv_barrier<0>();
    };
    // an interleaved iteration (n in 1 .. n_fast < n_end), slots by n % 3; its first
    // operands arrive in kpre / vpre and it leaves those of iteration n+1's first step
    // (K of tile n+1, V of tile n: stable across the barrier) in them
    u32x4 kpre[AHEAD], vpre[AHEAD];
    auto titer_fast = [&](int n, const unsigned char *Kn, const unsigned char *Kn1, const unsigned char *Vm,
                          unsigned char *Kw, unsigned char *Vw) __attribute__((always_inline)) {
        copies(n, Kw, Vw);
        step_full(Kn + BK * TL::ROWB, Vm + BK * TL::ROWB, Kn1, Kn, s0, s1, pb1, pb0, kpre, vpre);
        step_full(Kn1, Kn, Kn1 + BK * TL::ROWB, Kn + BK * TL::ROWB, s1, s0, pb0, pb1, kpre, vpre);
        kv_barrier<0>();
    };
    // one pass over the key tiles
    auto run = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] = f32x16{};
        l_run = 0.f;
        failed = false;
        if (N > 0) load_rows(kg, p.k_ss, kgo, 0, k0s);
        kv_barrier<0>();
        titer_seq(-1);
        titer_seq(0);
        int n = 1;
        // the interleaved iterations, three per trip so that every slot is static; the
        // first one's operands: K of tile 1 and V of tile 0, upper halves
        if (n_fast >= 1) {
#pragma unroll
            for (int i = 0; i < AHEAD; ++i) {
                kpre[i] = kfrag(k1s + BK * TL::ROWB, i);
                vpre[i] = vfrag(k0s + BK * TL::ROWB, i);
            }
        }
        while (n <= n_fast) {
            titer_fast(n, k1s, k2s, k0s, k0s, k2s);
            if (++n > n_fast) break;
            titer_fast(n, k2s, k0s, k1s, k1s, k0s);
            if (++n > n_fast) break;
            titer_fast(n, k0s, k1s, k2s, k2s, k1s);
            ++n;
        }
        for (; n <= n_end; ++n) titer_seq(n);
    };
    // the copies and barriers of one pass, computing nothing
    auto run_idle = [&]() __attribute__((always_inline)) {
        if (N > 0) load_rows(kg, p.k_ss, kgo, 0, k0s);
        kv_barrier<0>();
        for (int n = -1; n <= n_end; ++n) {
            const int r = (n + 3) % 3, r1 = r == 2 ? 0 : r + 1, r2 = r == 0 ? 2 : r - 1;
            copies(n, smem + r2 * TILEB, smem + r1 * TILEB);
            if (n < n_end) kv_barrier<0>();
        }
    };
    // staged: every wave of the workgroup is past its last tile, so the LDS is free: the
    // wave writes its 32 rows of O into its own slice (K tile layout) and stores whole
    // rows, 16 bytes per lane, instead of 8 bytes in each of 32 rows per instruction
    auto epilogue = [&](bool staged) __attribute__((always_inline)) {
        const float l_tot = l_run + __shfl_xor(l_run, 32);
        bool dropped = false;
        if (p.rowdrop) {
            const uint32_t rid = (uint32_t)(((int64_t)b * p.Hq + h) * p.Sq + row);
            dropped = fmix32(p.rd_seed ^ rid) < p.rd_thr;
        }
        const bool live = l_tot > 0.f && !dropped;
        const float inv = live ? 1.f / l_tot : 0.f;
        if (staged) {
            unsigned char *os = smem + wave_s * 32 * TL::ROWB;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 x = {oacc[db][4 * g4 + 0] * inv, oacc[db][4 * g4 + 1] * inv,
                                     oacc[db][4 * g4 + 2] * inv, oacc[db][4 * g4 + 3] * inv};
                    *(typename TT::vec4 *)(os + TL::off(l32, 4 * db + g4) + 8 * hi) = cvt4(x, TT{});
                }
            }
            constexpr int RPS = 64 / TL::CH;  // rows per store instruction
            uint16_t *ob = (uint16_t *)p.o + b * p.o_sb + h * p.o_sh;
#pragma unroll
            for (int i = 0; i < 32 / RPS; ++i) {
                const int rr = i * RPS + lane / TL::CH, c = lane % TL::CH;
                const u32x4 y = *(const u32x4 *)(os + TL::off(rr, c));
                if (r0 + rr < p.Sq) *(u32x4 *)(ob + (int64_t)(r0 + rr) * p.o_ss + 8 * c) = y;
            }
            if (row < p.Sq && hi == 0 && p.lse)
                p.lse[((int64_t)b * p.Hq + h) * p.Sq + row] = live ? (m_run + __log2f(l_tot)) * kLn2 : -INFINITY;
        } else if (row < p.Sq) {
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
    };

    // each row's exact max over its keys (for the waves whose first pass failed)
    auto run_max = [&]() __attribute__((always_inline)) {
        if (N > 0) load_rows(kg, p.k_ss, kgo, 0, k0s);
        kv_barrier<0>();
        float mloc = -INFINITY;
        for (int n = -1; n <= n_end; ++n) {
            const int r = (n + 3) % 3, r1 = r == 2 ? 0 : r + 1, r2 = r == 0 ? 2 : r - 1;
            copies(n, smem + r2 * TILEB, smem + r1 * TILEB);
#pragma unroll
            for (int hb = 0; hb < 2; ++hb) {
                const int u = 2 * n + hb;
                if (u >= 0 && u < Nbw) {
                    qk_seq(smem + r * TILEB + hb * BK * TL::ROWB, s0);
#pragma unroll
                    for (int e = 0; e < 16; ++e) mloc = fmaxf(mloc, masked_t(u, s0, e));
                }
            }
            if (n < n_end) kv_barrier<0>();
        }
        m_run = row_max2(mloc);
    };

    if (tid == 0) wg_failed = 0;  // ordered before its uses by the pass's first barrier
    m_run = -INFINITY;
    run();
    // did any wave of the workgroup fail? (every wave's last reads of the pass are done
    // after this barrier, so the next pass may refill the slots)
    if (failed && lane == 0) wg_failed = 1;
    kv_barrier<0>();
    const bool again = wg_failed != 0;
    if (!failed) epilogue(!again);
    if (again) {
        if (failed) {
            run_max();
            kv_barrier<0>();
            run();
            epilogue(false);
        } else {
            run_idle();
            kv_barrier<0>();
            run_idle();
        }
    }
}

}  // namespace mm
