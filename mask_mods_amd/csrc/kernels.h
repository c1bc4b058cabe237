// kernels.h -- parameter blocks and launchers shared between the C-ABI layer (api.cpp)
// and the kernel translation units. Host-visible; no device code here.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mm {

enum { MASK_CAUSAL = 1, MASK_WINDOW = 2, MASK_BLOCK = 4, MASK_DOC = 8 };

// Whether a causal forward starts its heaviest tiles first: not with a window, whose
// tiles carry equal work and are better run side by side, neighbours of one (b, h) on
// one XCD, so that the K/V they share is served by its L2 (3-4% at window 256). Packed
// documents keep the causal order (10% faster than side by side at 16 documents, forward
// and backward); the backward keeps it with a window too.
constexpr bool longest_first(int mask) { return (mask & MASK_CAUSAL) && !(mask & MASK_WINDOW); }

// block-mask granularity: query rows x keys per block
constexpr int kBlockQ = 128, kBlockKV = 64;

// Forward attention, one launch. Strides are in elements.
struct FwdParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int B, Hq, Hkv, Sq, Skv, group;
    int64_t q_sb, q_sh, q_ss;
    int64_t k_sb, k_sh, k_ss;
    int64_t v_sb, v_sh, v_ss;
    int64_t o_sb, o_sh, o_ss;
    float scale_log2;      // scale * log2(e): scores are kept in base-2 units
    const float *slopes;   // alibi slopes per query head (natural units) or nullptr
    int window;            // MASK_WINDOW half width
    int rowdrop;           // nonzero: rows with fmix32(seed ^ row) < thr are fully masked
    uint32_t rd_seed, rd_thr;
    int n_qtiles;          // query tiles per (b, h)
    const uint8_t *bm;     // block mask or nullptr: byte b*bm_sb + h*bm_sh + qblk*bm_sq + kblk
    int64_t bm_sb, bm_sh, bm_sq;
    float v_descale;       // fp8 inputs: V dequantisation factor (the Q/K ones are in scale_log2)
    const int32_t *qdoc, *kvdoc;  // document ids (non-decreasing per sequence) or nullptr
    int64_t qdoc_sb, kvdoc_sb;
};

// Backward (dQ, dK, dV). Strides are in elements.
struct BwdParams {
    const void *q, *k, *v, *o, *dout;
    const float *lse;      // forward LSE, natural log, [B, Hq, Sq] contiguous
    void *dq, *dk, *dv;
    float *ws_lse2;        // [B, Hq, sq_pad]: LSE * log2(e), +inf for rows with no kept key
    float *ws_nd;          // [B, Hq, sq_pad]: -D = -rowsum(dO * O)
    int B, Hq, Hkv, Sq, Skv, group;
    int sq_pad;            // Sq rounded up to a multiple of kBwdRowPad (rows of the workspace arrays)
    int64_t q_sb, q_sh, q_ss, k_sb, k_sh, k_ss, v_sb, v_sh, v_ss, o_sb, o_sh, o_ss;
    int64_t do_sb, do_sh, do_ss, dq_sb, dq_sh, dq_ss, dk_sb, dk_sh, dk_ss, dv_sb, dv_sh, dv_ss;
    float scale, scale_log2;
    const float *slopes;   // alibi slopes per query head (natural units) or nullptr
    int window;
    const uint8_t *bm;     // block mask or nullptr (as FwdParams)
    int64_t bm_sb, bm_sh, bm_sq;
    int n_tiles;           // q tiles (dQ kernel) or key tiles (dK/dV kernel) per head
    const int32_t *qdoc, *kvdoc;  // document ids (non-decreasing per sequence) or nullptr
    int64_t qdoc_sb, kvdoc_sb;
};

// Decode split pass + merge. Strides are in elements.
struct DecParams {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const uint16_t *mask;  // f16 additive mask or nullptr
    const int32_t *lens;   // per-sequence lengths or nullptr
    int B, Hq, Hkv, kv_len, group, splits, chunk;
    int64_t q_sb, q_sh;
    int64_t kv_sb, kv_sh, kv_ss;
    int64_t o_sb, o_sh;
    int64_t m_sb, m_sh;
    float scale_log2;
    float *ws_o;           // [B, Hq, splits, D] unnormalised partial outputs
    float *ws_m;           // [B, Hq, splits] partial row max (base 2)
    float *ws_l;           // [B, Hq, splits] partial row sum
    int heads_per_wg;      // query heads per split workgroup (1, 2 or 4; divides group)
    const int32_t *block_table;  // paged caches: [B, max_pages] page ids, or nullptr
    int64_t bt_sb;         // block-table row stride (elements)
    int page_shift;        // log2(page_size)
};

// Decode split pass: steps of keys in flight per loop iteration (8 with up to 2 query
// heads per workgroup, 4 with 4: the registers hold G queries and outputs), and the
// keys one iteration of a workgroup covers (4 waves, D/8 lanes per key). The host makes
// split chunks whole multiples of it, so no iteration runs partly empty.
constexpr int decode_steps_in_flight(int G) { return G <= 2 ? 8 : 4; }
constexpr int decode_iter_keys(int D, int G) { return 4 * (64 / (D / 8)) * decode_steps_in_flight(G); }

// Smallest number of query rows per forward workgroup (host-side grid bound).
constexpr int kFwdBM = 128;

// dtype: 1 = f16, 2 = bf16 (the mm_dtype values)
hipError_t launch_fwd_mfma_bf16_d64(const FwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_fwd_mfma_bf16_d128(const FwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_fwd_mfma_f16_d64(const FwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_fwd_mfma_f16_d128(const FwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_fwd_fp8_d64(const FwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_fwd_fp8_d128(const FwdParams &p, bool alibi, int mask, hipStream_t s);
hipError_t launch_fwd_f32(const FwdParams &p, int D, bool alibi, int mask, hipStream_t s);
hipError_t launch_decode(const DecParams &p, int dtype, int D, hipStream_t s);
// the three backward launches (pre-pass, dQ, dK/dV); dtype 1 = f16, 2 = bf16
hipError_t launch_bwd(const BwdParams &p, int dtype, int D, bool alibi, int mask, hipStream_t s);
constexpr int kBwdRowPad = 64;  // workspace rows per (b, h) are padded to this multiple
// window < 0: no window predicate
hipError_t launch_block_mask(uint8_t *out, int64_t ld, int Sq, int Skv, bool causal, int window,
                             hipStream_t s);

}  // namespace mm
