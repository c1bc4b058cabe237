// decode.hip -- one-query-per-head attention against a KV cache (split-KV, two passes).
//
// The decode form of IREE issue #19015 (example IR): q [B,H,1,D], K/V with a length
// known only at run time, an f16 scale and an additive f16 mask [B,H,1,L] added to the
// scaled score, accumulation in f32, output in the input type. With one query per head
// there are only B*H rows, far fewer than the 256 CUs, so the key range is cut into
// `splits` chunks and each (split, head, batch) gets its own workgroup:
//
//   pass 1 (split): stream the chunk's K/V rows from HBM with 16-byte coalesced,
//     non-temporal loads (D/8 lanes per key, 8 keys in flight per lane group), dot
//     products in fp32 (v_dot2 on the 16-bit inputs) reduced across the key's lanes
//     with DPP row ops, online softmax, and write the unnormalised partial output plus
//     its (max, sum) to the workspace;
//   pass 2 (merge): per (b, h) rescale the partials to the common max and normalise:
//     O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, LSE = (M + log2 L) ln 2.
// A row with no visible key (empty sequence or all -inf mask) yields O = 0, LSE = -inf.
// With GQA a workgroup serves up to 4 query heads of a kv head (all of a group of 2 or
// 4), so each K/V byte is read once per 4 heads; with a page table the K/V rows are
// gathered page by page.
#include "common.h"
#include "kernels.h"

namespace mm {

// Sum over each aligned group of N lanes (N = 8 or 16) with DPP row operations; every
// lane of the group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 8 || N == 16, "group");
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
    if (N == 16)
        v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x140, 0xF, 0xF, true));
    return v;
}

// q.k over the lane's 8 dims in fp32 (products of 16-bit values are exact in fp32)
__device__ __forceinline__ float dot8(u32x4 q, u32x4 k, F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // copy the elements out first: a bit_cast of a vector-element lvalue reads element 0
        const uint32_t qi = q[i], ki = k[i];
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, qi), __builtin_bit_cast(h2, ki), acc, false);
    }
    return acc;
}
__device__ __forceinline__ float dot8(u32x4 q, u32x4 k, BF16) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t qi = q[i], ki = k[i];
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, qi), __builtin_bit_cast(b2, ki), acc, false);
    }
    return acc;
}

// One workgroup = (split, group of G query heads sharing one kv head, batch). The G
// heads' queries sit in registers, so each K/V byte is read from HBM once for all of
// them (GQA); G = 1 is the plain per-head case. PAGED: key j of sequence b lives in
// page block_table[b][j / page_size], row j % page_size, of the K/V page pools.
template <typename TT, int D, bool MASKED, int G, bool PAGED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecParams p) {
    constexpr int LPK = D / 8;       // lanes per key (16 bytes each)
    constexpr int KPW = 64 / LPK;    // keys per wave per step
    constexpr int NW = 4;
    constexpr int STEP = NW * KPW;   // keys per workgroup per step
    constexpr int U = decode_steps_in_flight(G);  // steps in flight per iteration
    constexpr int SLOTS = NW * KPW;  // partial softmax states per workgroup and head
    static_assert(STEP * U == decode_iter_keys(D, G), "iteration size shared with the host");
    static_assert(G == 1 || G == 2 || G == 4, "heads per workgroup");

    __shared__ float sm_m[SLOTS], sm_l[SLOTS];
    __shared__ __attribute__((aligned(16))) float sm_o[SLOTS][D];

    const int hg = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / LPK, c = lane % LPK;
    const int slot = wave * KPW + g;
    const int h0 = hg * G;           // first query head of this workgroup
    const int hk = h0 / p.group;     // G divides the group: one kv head for all G
    // Workgroups go to the 8 XCDs round-robin by linear id, split index fastest. The
    // split index is rotated by the (batch, kv head) index, so that the first splits of
    // the rows (the only non-empty ones of a short sequence) spread over the XCDs
    // instead of all landing on one; the workgroups of one kv head keep the same
    // rotation, so those that read the same chunk still share an XCD.
    const int s = (int)(((int64_t)blockIdx.x + (int64_t)b * p.Hkv + hk) % p.splits);

    int len = p.kv_len;
    if (p.lens) len = min(max(p.lens[b], 0), p.kv_len);
    const int j_begin = s * p.chunk;
    const int j_end = min(len, j_begin + p.chunk);
    if (j_begin >= j_end) {
        // an empty split (a short sequence, or the rounded-up tail): weight 0 in the
        // merge, which then reads neither its output partial nor anything else of it.
        // With one split the row is empty: O = 0, LSE = -inf, written here.
        if (p.splits == 1) {
            for (int i = tid; i < G * D; i += 256) {
                const int gi = i / D, d = i % D;
                ((uint16_t *)p.o + b * p.o_sb + (h0 + gi) * p.o_sh)[d] = narrow1(0.f, TT{});
                if (d == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h0 + gi] = -INFINITY;
            }
        } else if (tid < G) {
            const int64_t wi = ((int64_t)b * p.Hq + h0 + tid) * p.splits + s;
            p.ws_m[wi] = -INFINITY;
            p.ws_l[wi] = 0.f;
        }
        return;
    }

    u32x4 qv[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
        qv[gi] = *(const u32x4 *)((const uint16_t *)p.q + b * p.q_sb + (h0 + gi) * p.q_sh + 8 * c);
    const float c2 = p.scale_log2;

    // contiguous caches: [B, Hkv, S, D]; page pools: [pages, Hkv, page_size, D]
    const uint16_t *kbase = (const uint16_t *)p.k + (PAGED ? 0 : b * p.kv_sb) + hk * p.kv_sh + 8 * c;
    const uint16_t *vbase = (const uint16_t *)p.v + (PAGED ? 0 : b * p.kv_sb) + hk * p.kv_sh + 8 * c;
    const int32_t *bt = PAGED ? p.block_table + b * p.bt_sb : nullptr;
    // page tables: the pages of an iteration's keys (the same keys as the loads below)
    // are read one iteration ahead, so the K/V loads never wait on a table read
    int32_t pg[U];
    if (PAGED && j_begin < j_end) {
#pragma unroll
        for (int u = 0; u < U; ++u) pg[u] = bt[min(j_begin + u * STEP + slot, j_end - 1) >> p.page_shift];
    }

    float m[G], l[G];
    f32x8 o[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        m[gi] = -INFINITY;
        l[gi] = 0.f;
        o[gi] = f32x8{};
    }

    // one iteration's loads: K/V rows of its U steps (and the G heads' mask entries);
    // then the page table entries of the next iteration
    auto load_iter = [&](int base, u32x4 (&kr)[U], u32x4 (&vr)[U], uint16_t (&mk)[U][G])
        __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = min(base + u * STEP + slot, j_end - 1);  // tail lanes re-read a valid key
            const int64_t off = PAGED ? (int64_t)pg[u] * p.kv_sb + (int64_t)(j & ((1 << p.page_shift) - 1)) * p.kv_ss
                                      : (int64_t)j * p.kv_ss;
            kr[u] = __builtin_nontemporal_load((const u32x4 *)(kbase + off));
            vr[u] = __builtin_nontemporal_load((const u32x4 *)(vbase + off));
            if (MASKED) {
#pragma unroll
                for (int gi = 0; gi < G; ++gi) mk[u][gi] = p.mask[b * p.m_sb + (h0 + gi) * p.m_sh + j];
            }
        }
        if (PAGED && base + STEP * U < j_end) {
#pragma unroll
            for (int u = 0; u < U; ++u) pg[u] = bt[min(base + STEP * U + u * STEP + slot, j_end - 1) >> p.page_shift];
        }
    };
    // online softmax over one iteration's keys for each of the G heads
    auto consume = [&](int base, const u32x4 (&kr)[U], const u32x4 (&vr)[U], const uint16_t (&mk)[U][G])
        __attribute__((always_inline)) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            float t[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float dot = group_sum<LPK>(dot8(qv[gi], kr[u], TT{})) * c2;
                if (MASKED) dot = fmaf(widen1(mk[u][gi], F16{}), kLog2e, dot);
                t[u] = base + u * STEP + slot < j_end ? dot : -INFINITY;
            }
            float mt = t[0];
#pragma unroll
            for (int u = 1; u < U; ++u) mt = fmaxf(mt, t[u]);
            const float m_new = fmaxf(m[gi], mt);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float alpha = fast_exp2(m[gi] - m_use);
            l[gi] *= alpha;
            o[gi] *= alpha;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float pv = fast_exp2(t[u] - m_use);
                l[gi] += pv;
                o[gi] += pv * widen8(vr[u], TT{});
            }
            m[gi] = m_new;
        }
    };

    for (int base = j_begin; base < j_end; base += STEP * U) {
        u32x4 kr[U], vr[U];
        uint16_t mk[U][G];
        load_iter(base, kr, vr, mk);
        consume(base, kr, vr, mk);
    }

    // combine the SLOTS partial states of each head (one head at a time through LDS)
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
        if (gi > 0) __syncthreads();  // the previous head's reads are done
        if (c == 0) {
            sm_m[slot] = m[gi];
            sm_l[slot] = l[gi];
        }
        *(f32x4 *)&sm_o[slot][8 * c] = f32x4{o[gi][0], o[gi][1], o[gi][2], o[gi][3]};
        *(f32x4 *)&sm_o[slot][8 * c + 4] = f32x4{o[gi][4], o[gi][5], o[gi][6], o[gi][7]};
        __syncthreads();
        if (tid < D) {
            float M = -INFINITY;
#pragma unroll
            for (int k = 0; k < SLOTS; ++k) M = fmaxf(M, sm_m[k]);
            float Ls = 0.f, Od = 0.f;
            if (M != -INFINITY) {
#pragma unroll
                for (int k = 0; k < SLOTS; ++k) {
                    const float mk2 = sm_m[k];
                    const float w = mk2 == -INFINITY ? 0.f : fast_exp2(mk2 - M);
                    Ls += sm_l[k] * w;
                    Od += sm_o[k][tid] * w;
                }
            }
            if (p.splits == 1) {
                // one split: this is the whole row; normalise here as the merge would
                // (its weights are then exactly 1), and skip the merge launch
                const bool live = Ls > 0.f;
                ((uint16_t *)p.o + b * p.o_sb + (h0 + gi) * p.o_sh)[tid] = narrow1(live ? Od / Ls : 0.f, TT{});
                if (tid == 0 && p.lse)
                    p.lse[(int64_t)b * p.Hq + h0 + gi] = live ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
            } else {
                const int64_t wi = ((int64_t)b * p.Hq + h0 + gi) * p.splits + s;
                p.ws_o[wi * D + tid] = Od;
                if (tid == 0) {
                    p.ws_m[wi] = M;
                    p.ws_l[wi] = Ls;
                }
            }
        }
    }
}

// One workgroup per (b, h): weights of all splits in parallel, then the weighted sum
// over splits split across 256 threads (D dims x 256/D split groups).
template <typename TT, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecParams p) {
    constexpr int SG = 256 / D;  // split groups
    __shared__ float sm_w[256];
    __shared__ float sm_red[2][4];
    __shared__ float sm_acc[SG][D];
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int64_t w0 = ((int64_t)b * p.Hq + h) * p.splits;
    const int S = p.splits;  // <= 256

    const float ms = tid < S ? p.ws_m[w0 + tid] : -INFINITY;
    const float ls = tid < S ? p.ws_l[w0 + tid] : 0.f;
    float M = ms;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
    if (lane == 0) sm_red[0][wave] = M;
    __syncthreads();
    M = fmaxf(fmaxf(sm_red[0][0], sm_red[0][1]), fmaxf(sm_red[0][2], sm_red[0][3]));
    const float w = (ms == -INFINITY || M == -INFINITY) ? 0.f : fast_exp2(ms - M);
    sm_w[tid] = w;
    float Lp = ls * w;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) Lp += __shfl_xor(Lp, off);
    if (lane == 0) sm_red[1][wave] = Lp;
    __syncthreads();
    const float Ls = sm_red[1][0] + sm_red[1][1] + sm_red[1][2] + sm_red[1][3];

    const int d = tid % D, sg = tid / D;
    const float *op0 = p.ws_o + w0 * D + d;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int s0 = sg;
    // a split of weight 0 (empty, or every key masked) is not read: an empty split
    // leaves its output partial unwritten. The weight test is uniform over each wave
    // (a wave's lanes share sg), so skipped loads cost no memory traffic.
    for (; s0 + 7 * SG < S; s0 += 8 * SG) {  // 8 independent loads in flight
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float wu = sm_w[s0 + u * SG];
            const float ou = wu != 0.f ? op0[(int64_t)(s0 + u * SG) * D] : 0.f;
            acc[u] = fmaf(wu, ou, acc[u]);
        }
    }
    for (; s0 < S; s0 += SG) {
        const float wu = sm_w[s0];
        acc[0] = fmaf(wu, wu != 0.f ? op0[(int64_t)s0 * D] : 0.f, acc[0]);
    }
    sm_acc[sg][d] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
    __syncthreads();
    if (tid < D) {
        float Od = 0.f;
#pragma unroll
        for (int g2 = 0; g2 < SG; ++g2) Od += sm_acc[g2][tid];
        const bool live = Ls > 0.f;
        uint16_t *op = (uint16_t *)p.o + b * p.o_sb + h * p.o_sh;
        op[tid] = narrow1(live ? Od / Ls : 0.f, TT{});
        if (tid == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h] = live ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
    }
}

template <typename TT, int D, int G, bool PAGED>
static hipError_t launch_split(const DecParams &p, hipStream_t s) {
    const dim3 g1((unsigned)p.splits, (unsigned)(p.Hq / G), (unsigned)p.B);
    if (p.mask)
        decode_split_kernel<TT, D, true, G, PAGED><<<g1, dim3(256), 0, s>>>(p);
    else
        decode_split_kernel<TT, D, false, G, PAGED><<<g1, dim3(256), 0, s>>>(p);
    return hipGetLastError();
}

template <typename TT, int D>
static hipError_t launch_decode_t(const DecParams &p, hipStream_t s) {
    hipError_t e;
    const bool paged = p.block_table != nullptr;
    switch (p.heads_per_wg) {
        case 4: e = paged ? launch_split<TT, D, 4, true>(p, s) : launch_split<TT, D, 4, false>(p, s); break;
        case 2: e = paged ? launch_split<TT, D, 2, true>(p, s) : launch_split<TT, D, 2, false>(p, s); break;
        default: e = paged ? launch_split<TT, D, 1, true>(p, s) : launch_split<TT, D, 1, false>(p, s); break;
    }
    if (e != hipSuccess || p.splits == 1) return e;  // one split writes the output itself
    decode_merge_kernel<TT, D><<<dim3((unsigned)p.Hq, (unsigned)p.B), dim3(256), 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecParams &p, int dtype, int D, hipStream_t s) {
    if (dtype == 2) return D == 64 ? launch_decode_t<BF16, 64>(p, s) : launch_decode_t<BF16, 128>(p, s);
    return D == 64 ? launch_decode_t<F16, 64>(p, s) : launch_decode_t<F16, 128>(p, s);
}

}  // namespace mm
