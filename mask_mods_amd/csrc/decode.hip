// decode.hip -- one-query-per-head attention against a KV cache (split-KV, two passes).
//
// The decode form of IREE issue #19015 (example IR): q [B,H,1,D], K/V with a length
// known only at run time, an f16 scale and an additive f16 mask [B,H,1,L] added to the
// scaled score, accumulation in f32, output in the input type. With one query per head
// there are only B*H rows, far fewer than the 256 CUs, so the key range is cut into
// `splits` chunks and each (split, head, batch) gets its own workgroup:
//
//   pass 1 (split): stream the chunk's K/V rows from HBM with 16-byte coalesced loads
//     (D/8 lanes per key, 4 keys in flight per lane group), dot products in fp32
//     reduced across the key's lanes, online softmax, and write the unnormalised
//     partial output plus its (max, sum) to the workspace;
//   pass 2 (merge): per (b, h) rescale the partials to the common max and normalise:
//     O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, LSE = (M + log2 L) ln 2.
// A row with no visible key (empty sequence or all -inf mask) yields O = 0, LSE = -inf.
#include "common.h"
#include "kernels.h"

namespace mm {

template <typename TT, int D, bool MASKED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecParams p) {
    constexpr int LPK = D / 8;       // lanes per key
    constexpr int KPW = 64 / LPK;    // keys per wave per step
    constexpr int NW = 4;
    constexpr int STEP = NW * KPW;   // keys per workgroup per step
    constexpr int U = 4;             // steps in flight per iteration
    constexpr int SLOTS = NW * KPW;  // partial softmax states per workgroup

    __shared__ float sm_m[SLOTS], sm_l[SLOTS];
    __shared__ __attribute__((aligned(16))) float sm_o[SLOTS][D];

    const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane / LPK, c = lane % LPK;
    const int slot = wave * KPW + g;
    const int hk = h / p.group;

    int len = p.kv_len;
    if (p.lens) len = min(max(p.lens[b], 0), p.kv_len);
    const int j_begin = s * p.chunk;
    const int j_end = min(len, j_begin + p.chunk);

    const uint16_t *qp = (const uint16_t *)p.q + b * p.q_sb + h * p.q_sh + 8 * c;
    f32x8 qf = widen8(*(const u32x4 *)qp, TT{}) * p.scale_log2;

    const uint16_t *kbase = (const uint16_t *)p.k + b * p.kv_sb + hk * p.kv_sh + 8 * c;
    const uint16_t *vbase = (const uint16_t *)p.v + b * p.kv_sb + hk * p.kv_sh + 8 * c;
    const uint16_t *mbase = MASKED ? p.mask + b * p.m_sb + h * p.m_sh : nullptr;

    float m = -INFINITY, l = 0.f;
    f32x8 o = {};

    for (int base = j_begin; base < j_end; base += STEP * U) {
        u32x4 kr[U], vr[U];
        uint16_t mk[U];
        bool valid[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = base + u * STEP + slot;
            valid[u] = j < j_end;
            kr[u] = valid[u] ? *(const u32x4 *)(kbase + (int64_t)j * p.kv_ss) : u32x4{0, 0, 0, 0};
            vr[u] = valid[u] ? *(const u32x4 *)(vbase + (int64_t)j * p.kv_ss) : u32x4{0, 0, 0, 0};
            if (MASKED) mk[u] = valid[u] ? mbase[j] : (uint16_t)0;
        }
        float t[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const f32x8 kf = widen8(kr[u], TT{});
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(qf[e], kf[e], dot);
#pragma unroll
            for (int off = LPK / 2; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
            if (MASKED) dot += widen1(mk[u], F16{}) * kLog2e;
            t[u] = valid[u] ? dot : -INFINITY;
        }
        float mt = t[0];
#pragma unroll
        for (int u = 1; u < U; ++u) mt = fmaxf(mt, t[u]);
        const float m_new = fmaxf(m, mt);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = fast_exp2(m - m_use);
        l *= alpha;
        o *= alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float pv = fast_exp2(t[u] - m_use);
            l += pv;
            o += pv * widen8(vr[u], TT{});
        }
        m = m_new;
    }

    if (c == 0) {
        sm_m[slot] = m;
        sm_l[slot] = l;
    }
    *(f32x4 *)&sm_o[slot][8 * c] = f32x4{o[0], o[1], o[2], o[3]};
    *(f32x4 *)&sm_o[slot][8 * c + 4] = f32x4{o[4], o[5], o[6], o[7]};
    __syncthreads();

    if (tid < D) {
        float M = -INFINITY;
#pragma unroll 8
        for (int k = 0; k < SLOTS; ++k) M = fmaxf(M, sm_m[k]);
        float Ls = 0.f, Od = 0.f;
        if (M != -INFINITY) {
            for (int k = 0; k < SLOTS; ++k) {
                const float mk2 = sm_m[k];
                const float w = mk2 == -INFINITY ? 0.f : fast_exp2(mk2 - M);
                Ls += sm_l[k] * w;
                Od += sm_o[k][tid] * w;
            }
        }
        const int64_t wi = ((int64_t)b * p.Hq + h) * p.splits + s;
        p.ws_o[wi * D + tid] = Od;
        if (tid == 0) {
            p.ws_m[wi] = M;
            p.ws_l[wi] = Ls;
        }
    }
}

template <typename TT, int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(DecParams p) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int64_t w0 = ((int64_t)b * p.Hq + h) * p.splits;
    float M = -INFINITY;
    for (int s = 0; s < p.splits; ++s) M = fmaxf(M, p.ws_m[w0 + s]);
    float Ls = 0.f, Od = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < p.splits; ++s) {
            const float ms = p.ws_m[w0 + s];
            const float w = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
            Ls += p.ws_l[w0 + s] * w;
            Od += p.ws_o[(w0 + s) * D + d] * w;
        }
    }
    const bool live = Ls > 0.f;
    const float val = live ? Od / Ls : 0.f;
    uint16_t *op = (uint16_t *)p.o + b * p.o_sb + h * p.o_sh;
    op[d] = narrow1(val, TT{});
    if (d == 0 && p.lse) p.lse[(int64_t)b * p.Hq + h] = live ? (M + __log2f(Ls)) * kLn2 : -INFINITY;
}

template <typename TT, int D>
static hipError_t launch_decode_t(const DecParams &p, hipStream_t s) {
    const dim3 g1((unsigned)p.splits, (unsigned)p.Hq, (unsigned)p.B);
    if (p.mask)
        decode_split_kernel<TT, D, true><<<g1, dim3(256), 0, s>>>(p);
    else
        decode_split_kernel<TT, D, false><<<g1, dim3(256), 0, s>>>(p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    decode_merge_kernel<TT, D><<<dim3((unsigned)p.Hq, (unsigned)p.B), dim3(D), 0, s>>>(p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecParams &p, int dtype, int D, hipStream_t s) {
    if (dtype == 2) return D == 64 ? launch_decode_t<BF16, 64>(p, s) : launch_decode_t<BF16, 128>(p, s);
    return D == 64 ? launch_decode_t<F16, 64>(p, s) : launch_decode_t<F16, 128>(p, s);
}

}  // namespace mm
