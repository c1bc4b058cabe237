// api.cpp -- the C ABI (include/maskmods.h): argument validation and dispatch.
//
// Every check runs on the host before anything is launched, so a rejected call has no
// effect on the device. Nothing here allocates device memory or keeps state.
#include "maskmods.h"

#include <math.h>

#include <atomic>
#include <mutex>

#include "kernels.h"

using namespace mm;

// The split partials of mm_attn_decode_noalloc: one static array per GPU, resident until
// the process ends. Host code never uses this name as an address (on the host it is
// only a stand-in); scratch_address() looks the device address up once per device.
static __device__ __align__(256) unsigned char scratch[MM_DECODE_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
std::atomic<void *> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device, looked up (with that device
// current) on the first call per device and kept; nullptr if the lookup fails or
// `stream` belongs to another device.
void *scratch_address(hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    if (stream) {
        hipDevice_t sdev = -1;
        if (hipStreamGetDevice(stream, &sdev) != hipSuccess || sdev != dev) return nullptr;
    }
    void *ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr) return ptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
        void *found = nullptr;
        if (hipGetSymbolAddress(&found, HIP_SYMBOL(scratch)) != hipSuccess || !found) return nullptr;
        g_scratch_ptr[dev].store(found, std::memory_order_release);
        ptr = found;
    }
    return ptr;
}

constexpr int kMaxSplits = 256;
constexpr int kMinKeysPerSplit = 256;
constexpr int kTargetDecodeBlocks = 1024;  // ~4 workgroups per CU, one resident round
constexpr int kVarlenGridFactor = 8;       // with per-sequence lengths: at most 8 rounds
// Sequence lengths stay below 2^30 so that the kernels' 32-bit index arithmetic (a row
// plus the window plus one, a key tile's end) cannot overflow.
constexpr int32_t kMaxSeq = 1 << 30;

// |q_idx - kv_idx| <= max(Sq, Skv) - 1 for every pair, so a window of max(Sq, Skv) keeps
// every pair exactly as any larger one does; clamping keeps the kernels' window
// arithmetic in range for windows up to INT32_MAX.
int32_t clamp_window(int32_t w, int32_t Sq, int32_t Skv) {
    const int32_t m = Sq > Skv ? Sq : Skv;
    return w > m ? m : w;
}

bool bad_strides(const int64_t *s, int n) {
    for (int i = 0; i < n; ++i)
        if (s[i] < 0) return true;
    return false;
}

// 16-byte vector loads/stores on the 16-bit paths: pointers 16-byte aligned and every
// stride a multiple of 8 elements.
bool misaligned16(const void *p) { return ((uintptr_t)p & 15u) != 0; }
bool strides_not_mult(const int64_t *s, int n, int m) {
    for (int i = 0; i < n; ++i)
        if (s[i] % m != 0) return true;
    return false;
}

// The document mask's id arrays: both present (when any pair exists), 4-byte aligned,
// non-negative strides.
mm_status check_doc(const mm_mods &m, bool pairs) {
    if (!(m.mask_flags & MM_MASK_DOCUMENT)) return MM_OK;
    if (pairs && (!m.q_doc_ids || !m.kv_doc_ids)) return MM_ERR_NULL;
    if (bad_strides(m.doc_strides, 2)) return MM_ERR_STRIDE;
    if (((uintptr_t)m.q_doc_ids | (uintptr_t)m.kv_doc_ids) & 3u) return MM_ERR_STRIDE;
    return MM_OK;
}

// Query heads per split workgroup: the largest of 4, 2, 1 that divides the group (a
// workgroup of 8 heads held too few loads in flight and ran slower than two of 4).
int decode_heads_per_wg(int32_t Hq, int32_t Hkv) {
    const int group = Hq / Hkv;
    for (int g = 4; g > 1; g >>= 1)
        if (group % g == 0) return g;
    return 1;
}

// splits: at most one resident round of (split, head group, batch) workgroups, rounded
// down so that no CU gets one workgroup more than the others: about 1024 with one head
// per workgroup, 512 with 2 or 4 (their registers leave room for 3 per CU, not 4); no
// split shorter than kMinKeysPerSplit keys; and, when a kv head's group spans several
// workgroups, a multiple of 8: workgroups are placed on the 8 XCDs round-robin by
// linear id (split fastest), so the workgroups that read the same K/V chunk then share
// one XCD's L2 instead of each fetching it from HBM.
// varlen (per-sequence lengths, known only on the device): one sequence may hold
// nearly all of the batch's keys, so the count is raised to what a batch of one would
// get, within a grid of kVarlenGridFactor resident rounds; the workgroups of the
// shorter sequences' empty splits end at once.
int decode_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t kv_len, int32_t requested, bool varlen) {
    if (requested > 0) return requested;
    if (kv_len <= 0) return 1;
    const int G = decode_heads_per_wg(Hq, Hkv);
    const int64_t rows = (int64_t)B * Hq / G;
    const int64_t target = G > 1 ? kTargetDecodeBlocks / 2 : kTargetDecodeBlocks;
    int64_t want = target / rows;
    if (varlen) {
        const int64_t one = target / (Hq / G);
        const int64_t cap = kVarlenGridFactor * target / rows;
        const int64_t raised = one < cap ? one : cap;
        if (raised > want) want = raised;
    }
    const int64_t by_len = ((int64_t)kv_len + kMinKeysPerSplit - 1) / kMinKeysPerSplit;
    if (want > by_len) want = by_len;
    if (want > kMaxSplits) want = kMaxSplits;
    if (Hq / Hkv > G && want >= 8) want = want / 8 * 8;
    if (want < 1) want = 1;
    return (int)want;
}

}  // namespace

extern "C" {

int32_t mm_version(void) { return 400; }

#ifndef MM_SOURCE_HASH
#define MM_SOURCE_HASH "unknown"
#endif
const char *mm_source_hash(void) { return MM_SOURCE_HASH; }

size_t mm_fwd_args_size(void) { return sizeof(mm_fwd_args); }
size_t mm_decode_args_size(void) { return sizeof(mm_decode_args); }
size_t mm_bwd_args_size(void) { return sizeof(mm_bwd_args); }

const char *mm_status_str(int32_t st) {
    switch (st) {
        case MM_OK: return "ok";
        case MM_ERR_NULL: return "required pointer is NULL";
        case MM_ERR_SHAPE: return "invalid shape";
        case MM_ERR_DTYPE: return "unsupported dtype";
        case MM_ERR_UNSUPPORTED: return "unsupported head dim or mod";
        case MM_ERR_STRIDE: return "invalid stride or alignment";
        case MM_ERR_LAUNCH: return "kernel launch failed";
        case MM_ERR_WORKSPACE: return "workspace missing or too small";
        default: return "unknown status";
    }
}

mm_status mm_attn_fwd(const mm_fwd_args *a, void *stream) {
    if (!a) return MM_ERR_NULL;
    // empty tensors may legitimately have NULL data pointers
    const bool no_rows = (int64_t)a->B * a->Hq * a->Sq == 0;
    if ((!a->q || !a->out) && !no_rows) return MM_ERR_NULL;
    if ((!a->k || !a->v) && (int64_t)a->B * a->Hkv * a->Skv != 0) return MM_ERR_NULL;
    if (a->dtype != MM_F32 && a->dtype != MM_F16 && a->dtype != MM_BF16 && a->dtype != MM_FP8_E4M3)
        return MM_ERR_DTYPE;
    const bool fp8 = a->dtype == MM_FP8_E4M3;
    if (fp8 && !(isfinite(a->descale_q) && isfinite(a->descale_k) && isfinite(a->descale_v) &&
                 a->descale_q > 0.f && a->descale_k > 0.f && a->descale_v > 0.f))
        return MM_ERR_SHAPE;
    if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Sq < 0 || a->Skv < 0) return MM_ERR_SHAPE;
    if (a->Sq >= kMaxSeq || a->Skv >= kMaxSeq) return MM_ERR_SHAPE;
    if (a->Hq % a->Hkv != 0) return MM_ERR_SHAPE;
    if (a->D != 64 && a->D != 128) return MM_ERR_UNSUPPORTED;
    if (a->mods.score_mod != MM_SCORE_NONE && a->mods.score_mod != MM_SCORE_ALIBI) return MM_ERR_UNSUPPORTED;
    if (a->mods.mask_flags & ~(uint32_t)(MM_MASK_CAUSAL | MM_MASK_WINDOW | MM_MASK_ROWDROP | MM_MASK_DOCUMENT))
        return MM_ERR_UNSUPPORTED;
    if ((a->mods.mask_flags & MM_MASK_WINDOW) && a->mods.window < 0) return MM_ERR_SHAPE;
    if (a->mods.block_mask && bad_strides(a->mods.block_mask_strides, 3)) return MM_ERR_STRIDE;
    if (const mm_status ds = check_doc(a->mods, !no_rows && (int64_t)a->B * a->Skv != 0)) return ds;
    if (!isfinite(a->scale)) return MM_ERR_SHAPE;
    if (bad_strides(a->q_strides, 3) || bad_strides(a->k_strides, 3) || bad_strides(a->v_strides, 3) ||
        bad_strides(a->o_strides, 3))
        return MM_ERR_STRIDE;
    if (a->dtype != MM_F32) {
        if (misaligned16(a->q) || misaligned16(a->k) || misaligned16(a->v) || misaligned16(a->out))
            return MM_ERR_STRIDE;
        // 16-byte vectors: 8 elements of 16 bits, 16 of fp8 (the bf16 output keeps 8)
        const int in_mult = fp8 ? 16 : 8;
        if (strides_not_mult(a->q_strides, 3, in_mult) || strides_not_mult(a->k_strides, 3, in_mult) ||
            strides_not_mult(a->v_strides, 3, in_mult) || strides_not_mult(a->o_strides, 3, 8))
            return MM_ERR_STRIDE;
        // the MFMA kernels address a 64-key tile with 32-bit byte offsets
        const int64_t esz = fp8 ? 1 : 2;
        if ((64 * a->k_strides[2] + a->D) * esz >= ((int64_t)1 << 31) ||
            (64 * a->v_strides[2] + a->D) * esz >= ((int64_t)1 << 31))
            return MM_ERR_STRIDE;
    } else {
        if (((uintptr_t)a->q | (uintptr_t)a->k | (uintptr_t)a->v | (uintptr_t)a->out) & 3u) return MM_ERR_STRIDE;
    }
    if (no_rows) return MM_OK;  // nothing to compute

    FwdParams p = {};
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.o = a->out;
    p.lse = a->lse;
    p.B = a->B;
    p.Hq = a->Hq;
    p.Hkv = a->Hkv;
    p.Sq = a->Sq;
    p.Skv = a->Skv;
    p.group = a->Hq / a->Hkv;
    p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_ss = a->q_strides[2];
    p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_ss = a->k_strides[2];
    p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_ss = a->v_strides[2];
    p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1]; p.o_ss = a->o_strides[2];
    p.scale_log2 = a->scale * 1.4426950408889634f;
    p.v_descale = 1.f;
    if (fp8) {
        p.scale_log2 = (float)((double)a->scale * a->descale_q * a->descale_k * 1.4426950408889634);
        p.v_descale = a->descale_v;
    }
    p.slopes = a->mods.alibi_slopes;
    p.window = clamp_window(a->mods.window, a->Sq, a->Skv);
    p.rowdrop = (a->mods.mask_flags & MM_MASK_ROWDROP) ? 1 : 0;
    p.rd_seed = a->mods.rowdrop_seed;
    p.rd_thr = a->mods.rowdrop_threshold;
    p.bm = a->mods.block_mask;
    p.bm_sb = a->mods.block_mask_strides[0];
    p.bm_sh = a->mods.block_mask_strides[1];
    p.bm_sq = a->mods.block_mask_strides[2];
    static_assert(MM_BLOCK_Q == kBlockQ && MM_BLOCK_KV == kBlockKV, "block-mask granularity");

    int mask = 0;
    if (a->causal || (a->mods.mask_flags & MM_MASK_CAUSAL)) mask |= MASK_CAUSAL;
    if (a->mods.mask_flags & MM_MASK_WINDOW) mask |= MASK_WINDOW;
    if (a->mods.block_mask) mask |= MASK_BLOCK;
    // with no keys there is nothing to mask (and the ids may be absent)
    if ((a->mods.mask_flags & MM_MASK_DOCUMENT) && a->Skv > 0) mask |= MASK_DOC;
    p.qdoc = a->mods.q_doc_ids;
    p.kvdoc = a->mods.kv_doc_ids;
    p.qdoc_sb = a->mods.doc_strides[0];
    p.kvdoc_sb = a->mods.doc_strides[1];
    const bool alibi = a->mods.score_mod == MM_SCORE_ALIBI;
    hipStream_t s = (hipStream_t)stream;

    hipError_t e;
    if (a->dtype == MM_F32) {
        p.n_qtiles = 1;
        e = launch_fwd_f32(p, a->D, alibi, mask, s);
    } else {
        if ((int64_t)((a->Sq + kFwdBM - 1) / kFwdBM) * a->Hq * a->B > 0x7fffffff) return MM_ERR_SHAPE;
        if (fp8)
            e = a->D == 64 ? launch_fwd_fp8_d64(p, alibi, mask, s) : launch_fwd_fp8_d128(p, alibi, mask, s);
        else if (a->dtype == MM_BF16)
            e = a->D == 64 ? launch_fwd_mfma_bf16_d64(p, alibi, mask, s) : launch_fwd_mfma_bf16_d128(p, alibi, mask, s);
        else
            e = a->D == 64 ? launch_fwd_mfma_f16_d64(p, alibi, mask, s) : launch_fwd_mfma_f16_d128(p, alibi, mask, s);
    }
    return e == hipSuccess ? MM_OK : MM_ERR_LAUNCH;
}

mm_status mm_block_mask_create(uint32_t mask_flags, int32_t window, int32_t Sq, int32_t Skv, uint8_t *out,
                               int64_t ld, void *stream) {
    if (mask_flags & ~(uint32_t)(MM_MASK_CAUSAL | MM_MASK_WINDOW)) return MM_ERR_UNSUPPORTED;
    if (Sq < 0 || Skv < 0) return MM_ERR_SHAPE;
    if ((mask_flags & MM_MASK_WINDOW) && window < 0) return MM_ERR_SHAPE;
    const int64_t nkb = ((int64_t)Skv + MM_BLOCK_KV - 1) / MM_BLOCK_KV;
    const int64_t nqb = ((int64_t)Sq + MM_BLOCK_Q - 1) / MM_BLOCK_Q;
    if (nkb == 0 || nqb == 0) return MM_OK;
    if (!out) return MM_ERR_NULL;
    if (ld < nkb) return MM_ERR_STRIDE;
    const hipError_t e = launch_block_mask(out, ld, Sq, Skv, (mask_flags & MM_MASK_CAUSAL) != 0,
                                           (mask_flags & MM_MASK_WINDOW) ? window : -1, (hipStream_t)stream);
    return e == hipSuccess ? MM_OK : MM_ERR_LAUNCH;
}

size_t mm_attn_bwd_workspace_size(int32_t B, int32_t Hq, int32_t Sq) {
    if (B < 0 || Hq <= 0 || Sq < 0) return 0;
    const int64_t pad = ((int64_t)Sq + kBwdRowPad - 1) / kBwdRowPad * kBwdRowPad;
    return (size_t)(2 * (int64_t)B * Hq * pad * (int64_t)sizeof(float));
}

mm_status mm_attn_bwd(const mm_bwd_args *a, void *stream) {
    if (!a) return MM_ERR_NULL;
    if (a->dtype != MM_F16 && a->dtype != MM_BF16) return MM_ERR_DTYPE;
    if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->Sq < 0 || a->Skv < 0) return MM_ERR_SHAPE;
    if (a->Sq >= kMaxSeq || a->Skv >= kMaxSeq) return MM_ERR_SHAPE;
    if (a->Hq % a->Hkv != 0) return MM_ERR_SHAPE;
    if (a->D != 64 && a->D != 128) return MM_ERR_UNSUPPORTED;
    const bool rows = (int64_t)a->B * a->Hq * a->Sq != 0, keys = (int64_t)a->B * a->Hkv * a->Skv != 0;
    if (rows && (!a->q || !a->out || !a->dout || !a->lse || !a->dq)) return MM_ERR_NULL;
    if (keys && (!a->k || !a->v || !a->dk || !a->dv)) return MM_ERR_NULL;
    if (a->mods.score_mod != MM_SCORE_NONE && a->mods.score_mod != MM_SCORE_ALIBI) return MM_ERR_UNSUPPORTED;
    if (a->mods.mask_flags & ~(uint32_t)(MM_MASK_CAUSAL | MM_MASK_WINDOW | MM_MASK_ROWDROP | MM_MASK_DOCUMENT))
        return MM_ERR_UNSUPPORTED;
    if ((a->mods.mask_flags & MM_MASK_WINDOW) && a->mods.window < 0) return MM_ERR_SHAPE;
    if (a->mods.block_mask && bad_strides(a->mods.block_mask_strides, 3)) return MM_ERR_STRIDE;
    if (const mm_status ds = check_doc(a->mods, rows && keys)) return ds;
    if (!isfinite(a->scale)) return MM_ERR_SHAPE;
    const int64_t *st[8] = {a->q_strides, a->k_strides, a->v_strides, a->o_strides,
                            a->do_strides, a->dq_strides, a->dk_strides, a->dv_strides};
    const void *ptr[8] = {a->q, a->k, a->v, a->out, a->dout, a->dq, a->dk, a->dv};
    for (int t = 0; t < 8; ++t) {
        if (bad_strides(st[t], 3) || strides_not_mult(st[t], 3, 8)) return MM_ERR_STRIDE;
        if (misaligned16(ptr[t])) return MM_ERR_STRIDE;
    }
    // 32-bit byte offsets inside a copied tile: 64 K/V rows, 32 Q/dO rows
    if ((64 * a->k_strides[2] + a->D) * 2 >= ((int64_t)1 << 31) ||
        (64 * a->v_strides[2] + a->D) * 2 >= ((int64_t)1 << 31) ||
        (32 * a->q_strides[2] + a->D) * 2 >= ((int64_t)1 << 31) ||
        (32 * a->do_strides[2] + a->D) * 2 >= ((int64_t)1 << 31))
        return MM_ERR_STRIDE;
    if (!rows && !keys) return MM_OK;
    const size_t need = mm_attn_bwd_workspace_size(a->B, a->Hq, a->Sq);
    if (rows && (!a->workspace || a->workspace_bytes < need)) return MM_ERR_WORKSPACE;
    if (((uintptr_t)a->workspace & 15u) != 0) return MM_ERR_WORKSPACE;
    if ((int64_t)((a->Sq + kFwdBM - 1) / kFwdBM) * a->Hq * a->B > 0x7fffffff ||
        (int64_t)((a->Skv + kFwdBM - 1) / kFwdBM) * a->Hkv * a->B > 0x7fffffff)
        return MM_ERR_SHAPE;

    BwdParams p = {};
    p.q = a->q; p.k = a->k; p.v = a->v; p.o = a->out; p.dout = a->dout; p.lse = a->lse;
    p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
    p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.Sq = a->Sq; p.Skv = a->Skv; p.group = a->Hq / a->Hkv;
    p.sq_pad = (a->Sq + kBwdRowPad - 1) / kBwdRowPad * kBwdRowPad;
    p.ws_lse2 = (float *)a->workspace;
    p.ws_nd = p.ws_lse2 + (int64_t)a->B * a->Hq * p.sq_pad;
    p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1]; p.q_ss = a->q_strides[2];
    p.k_sb = a->k_strides[0]; p.k_sh = a->k_strides[1]; p.k_ss = a->k_strides[2];
    p.v_sb = a->v_strides[0]; p.v_sh = a->v_strides[1]; p.v_ss = a->v_strides[2];
    p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1]; p.o_ss = a->o_strides[2];
    p.do_sb = a->do_strides[0]; p.do_sh = a->do_strides[1]; p.do_ss = a->do_strides[2];
    p.dq_sb = a->dq_strides[0]; p.dq_sh = a->dq_strides[1]; p.dq_ss = a->dq_strides[2];
    p.dk_sb = a->dk_strides[0]; p.dk_sh = a->dk_strides[1]; p.dk_ss = a->dk_strides[2];
    p.dv_sb = a->dv_strides[0]; p.dv_sh = a->dv_strides[1]; p.dv_ss = a->dv_strides[2];
    p.scale = a->scale;
    p.scale_log2 = a->scale * 1.4426950408889634f;
    p.slopes = a->mods.alibi_slopes;
    p.window = clamp_window(a->mods.window, a->Sq, a->Skv);
    p.bm = a->mods.block_mask;
    p.bm_sb = a->mods.block_mask_strides[0];
    p.bm_sh = a->mods.block_mask_strides[1];
    p.bm_sq = a->mods.block_mask_strides[2];
    int mask = 0;
    if (a->causal || (a->mods.mask_flags & MM_MASK_CAUSAL)) mask |= MASK_CAUSAL;
    if (a->mods.mask_flags & MM_MASK_WINDOW) mask |= MASK_WINDOW;
    if (a->mods.block_mask) mask |= MASK_BLOCK;
    // without rows or keys there is no pair to mask (and the ids may be absent)
    if ((a->mods.mask_flags & MM_MASK_DOCUMENT) && rows && keys) mask |= MASK_DOC;
    p.qdoc = a->mods.q_doc_ids;
    p.kvdoc = a->mods.kv_doc_ids;
    p.qdoc_sb = a->mods.doc_strides[0];
    p.kvdoc_sb = a->mods.doc_strides[1];
    // the row-drop mod needs nothing here: dropped rows have LSE = -inf
    const hipError_t e = launch_bwd(p, a->dtype, a->D, a->mods.score_mod == MM_SCORE_ALIBI, mask,
                                    (hipStream_t)stream);
    return e == hipSuccess ? MM_OK : MM_ERR_LAUNCH;
}

int32_t mm_attn_decode_auto_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t kv_len) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || kv_len < 0) return 0;
    return decode_splits(B, Hq, Hkv, kv_len, 0, false);
}

int32_t mm_attn_decode_auto_splits_varlen(int32_t B, int32_t Hq, int32_t Hkv, int32_t kv_len) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || kv_len < 0) return 0;
    return decode_splits(B, Hq, Hkv, kv_len, 0, true);
}

size_t mm_attn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t kv_len, int32_t D,
                                     int32_t num_splits) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || kv_len < 0 || (D != 64 && D != 128) ||
        num_splits < 0 || num_splits > kMaxSplits)
        return 0;
    const int splits = decode_splits(B, Hq, Hkv, kv_len, num_splits, true);  // >= the count without seq_lens
    return (size_t)B * Hq * splits * (size_t)(D + 2) * sizeof(float);
}

}  // extern "C"

namespace {

// mm_attn_decode and mm_attn_decode_noalloc: the same checks and launches; the second
// puts the partials in the static scratch instead of the caller's workspace.
mm_status decode_impl(const mm_decode_args *a, void *stream, bool static_scratch) {
    if (!a) return MM_ERR_NULL;
    if (a->B != 0 && (!a->q || !a->out)) return MM_ERR_NULL;
    if (a->B != 0 && a->kv_len > 0 && (!a->k_cache || !a->v_cache)) return MM_ERR_NULL;
    if (a->dtype != MM_F16 && a->dtype != MM_BF16) return MM_ERR_DTYPE;
    if (a->B < 0 || a->Hq <= 0 || a->Hkv <= 0 || a->kv_len < 0 || a->Scap < a->kv_len) return MM_ERR_SHAPE;
    if (a->Hq % a->Hkv != 0) return MM_ERR_SHAPE;
    if (a->D != 64 && a->D != 128) return MM_ERR_UNSUPPORTED;
    if (a->num_splits < 0 || a->num_splits > kMaxSplits) return MM_ERR_UNSUPPORTED;
    if (!isfinite(a->scale)) return MM_ERR_SHAPE;
    if (bad_strides(a->q_strides, 2) || bad_strides(a->kv_strides, 3) || bad_strides(a->o_strides, 2) ||
        bad_strides(a->mask_strides, 2))
        return MM_ERR_STRIDE;
    if (misaligned16(a->q) || misaligned16(a->k_cache) || misaligned16(a->v_cache))
        return MM_ERR_STRIDE;
    if (strides_not_mult(a->q_strides, 2, 8) || strides_not_mult(a->kv_strides, 3, 8)) return MM_ERR_STRIDE;
    if (((uintptr_t)a->out & 1u) || ((uintptr_t)a->mask & 1u)) return MM_ERR_STRIDE;
    int page_shift = 0;
    if (a->block_table) {
        if (a->page_size <= 0 || (a->page_size & (a->page_size - 1)) != 0) return MM_ERR_SHAPE;
        if (a->block_table_stride < 0) return MM_ERR_STRIDE;
        while ((1 << page_shift) < a->page_size) ++page_shift;
        if ((int64_t)(a->Scap + a->page_size - 1) / a->page_size > a->block_table_stride && a->B > 1)
            return MM_ERR_STRIDE;  // rows of the table would overlap
    }
    if (a->B == 0) return MM_OK;

    const int splits = decode_splits(a->B, a->Hq, a->Hkv, a->kv_len, a->num_splits, a->seq_lens != nullptr);
    const size_t need = (size_t)a->B * a->Hq * splits * (size_t)(a->D + 2) * sizeof(float);
    void *workspace = a->workspace;
    size_t workspace_bytes = a->workspace_bytes;
    if (static_scratch) {
        if (need > (size_t)MM_DECODE_SCRATCH_BYTES) return MM_ERR_WORKSPACE;
        workspace = scratch_address((hipStream_t)stream);
        if (!workspace) return MM_ERR_LAUNCH;
        workspace_bytes = MM_DECODE_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < need) return MM_ERR_WORKSPACE;
    if (misaligned16(workspace)) return MM_ERR_WORKSPACE;

    DecParams p = {};
    p.q = a->q;
    p.k = a->k_cache;
    p.v = a->v_cache;
    p.o = a->out;
    p.lse = a->lse;
    p.mask = (const uint16_t *)a->mask;
    p.lens = a->seq_lens;
    p.B = a->B;
    p.Hq = a->Hq;
    p.Hkv = a->Hkv;
    p.kv_len = a->kv_len;
    p.group = a->Hq / a->Hkv;
    p.splits = splits;
    p.chunk = a->kv_len > 0 ? (a->kv_len + splits - 1) / splits : 1;
    {
        // whole loop iterations per split (the last splits may then be empty)
        const int64_t it = decode_iter_keys(a->D, decode_heads_per_wg(a->Hq, a->Hkv));
        const int64_t aligned = (p.chunk + it - 1) / it * it;
        if (aligned * splits <= INT32_MAX) p.chunk = (int)aligned;
    }
    p.q_sb = a->q_strides[0]; p.q_sh = a->q_strides[1];
    p.kv_sb = a->kv_strides[0]; p.kv_sh = a->kv_strides[1]; p.kv_ss = a->kv_strides[2];
    p.o_sb = a->o_strides[0]; p.o_sh = a->o_strides[1];
    p.m_sb = a->mask_strides[0]; p.m_sh = a->mask_strides[1];
    p.scale_log2 = a->scale * 1.4426950408889634f;
    float *ws = (float *)workspace;
    const size_t nrow = (size_t)a->B * a->Hq * splits;
    p.ws_o = ws;
    p.ws_m = ws + nrow * a->D;
    p.ws_l = p.ws_m + nrow;
    p.heads_per_wg = decode_heads_per_wg(a->Hq, a->Hkv);
    p.block_table = a->block_table;
    p.bt_sb = a->block_table_stride;
    p.page_shift = page_shift;

    const hipError_t e = launch_decode(p, a->dtype, a->D, (hipStream_t)stream);
    return e == hipSuccess ? MM_OK : MM_ERR_LAUNCH;
}

}  // namespace

extern "C" {

mm_status mm_attn_decode(const mm_decode_args *a, void *stream) { return decode_impl(a, stream, false); }

mm_status mm_attn_decode_noalloc(const mm_decode_args *a, void *stream) { return decode_impl(a, stream, true); }

}  // extern "C"
