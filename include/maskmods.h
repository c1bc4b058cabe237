/*
 * maskmods.h -- C ABI of libmaskmods.so: fused flex-style attention for MI355X (gfx950).
 *
 * The operations, all asynchronous on the caller's HIP stream:
 *
 *   mm_attn_fwd     O = softmax(mask_mod(score_mod(scale * Q K^T))) V, plus the
 *                   row log-sum-exp. This is PyTorch's flex_attention operator as the
 *                   torch-mlir PR "[TORCH] Added flex_attention hop function" states
 *                   its operands (query, key, value, scale, enable_gqa, return_lse,
 *                   score_mod, mask_mod), with the built-in mods of FlyDSL PR #931
 *                   ("Add flex_attention (score_mod / mask_mod) on the generic
 *                   flash-attention kernel", Summary): alibi score_mod, causal and
 *                   sliding-window mask_mods, applied scale first, then score_mod,
 *                   then mask_mod; fully masked rows give O = 0 and LSE = -inf.
 *                   Beyond those: a row-drop mask_mod, a document mask_mod over
 *                   captured id tensors, block-sparse masks, fp8 (e4m3) inputs.
 *
 *   mm_attn_bwd     the gradients of that forward (dQ, dK, dV) for the same mods,
 *                   from its O and LSE: the backward the FlyDSL PR lists as a later
 *                   phase.
 *
 *   mm_attn_decode  one query per head against a KV cache whose length is known
 *                   only at run time, with an optional additive f16 mask: the
 *                   decode attention of IREE issue #19015 ("[ROCM] Support dynamic
 *                   key-value cache sequence length", example IR: Q [B,H,1,D],
 *                   K/V [B,H,?,D], f16 scale, mask [B,H,1,?], f32 score region),
 *                   extended to per-sequence lengths and paged caches (the issue
 *                   asks for a dynamic batch as well) and to GQA.
 *
 *   mm_block_mask_create  the block classes of the built-in predicates, for the
 *                   block-sparse path of mm_attn_fwd / mm_attn_bwd.
 *
 * Conventions shared by the calls
 *   - Tensors are row-major [B, H, S, D] with D innermost (stride 1). Strides are
 *     given in ELEMENTS for the b, h and s dimensions.
 *   - All tensor pointers are DEVICE pointers owned by the caller and borrowed for
 *     the call; they must stay valid until the work on `stream` completes. The
 *     library allocates no device memory and keeps no state between calls.
 *   - GQA: Hq must be a multiple of Hkv; query head h reads K/V head h / (Hq/Hkv).
 *   - Index alignment: q_idx and kv_idx are raw positions (top-left aligned when
 *     Sq != Skv).
 *   - LSE is natural-log, fp32, contiguous [B, Hq, Sq]; pass NULL to skip it.
 *   - Arguments are validated on the host before anything is launched; a rejected
 *     call launches nothing and returns a negative mm_status. A launch failure
 *     reported by the runtime returns MM_ERR_LAUNCH. Non-finite Q/K/V or a +inf/NaN
 *     mask entry give undefined results.
 *   - `stream` is a hipStream_t (NULL = the default stream).
 */
#ifndef MASKMODS_H
#define MASKMODS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MM_OK = 0,
    MM_ERR_NULL = -1,        /* a required pointer is NULL                      */
    MM_ERR_SHAPE = -2,       /* bad size (<=0, Hq % Hkv != 0, kv_len > Scap ...) */
    MM_ERR_DTYPE = -3,       /* dtype not supported by this call                */
    MM_ERR_UNSUPPORTED = -4, /* head dim or mod combination not built           */
    MM_ERR_STRIDE = -5,      /* D stride is not 1 or a stride is negative       */
    MM_ERR_LAUNCH = -6,      /* the HIP runtime reported a launch error         */
    MM_ERR_WORKSPACE = -7    /* decode workspace NULL or too small              */
} mm_status;

/* MM_FP8_E4M3: OCP 8-bit float (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
 * max 448; what torch calls float8_e4m3fn), forward only; the output is bf16. */
typedef enum { MM_F32 = 0, MM_F16 = 1, MM_BF16 = 2, MM_FP8_E4M3 = 3 } mm_dtype;

/* score_mod(score, b, h, q_idx, kv_idx) -> score, applied to the scaled score */
typedef enum {
    MM_SCORE_NONE = 0,
    MM_SCORE_ALIBI = 1 /* score + slope_h * (kv_idx - q_idx) */
} mm_score_mod;

/* mask_mod(b, h, q_idx, kv_idx) -> keep; flags are AND-composed */
enum {
    MM_MASK_NONE = 0u,
    MM_MASK_CAUSAL = 1u,  /* keep iff kv_idx <= q_idx                                  */
    MM_MASK_WINDOW = 2u,  /* keep iff |q_idx - kv_idx| <= window (inclusive)           */
    MM_MASK_ROWDROP = 4u, /* drop the whole row iff fmix32(seed ^ row) < threshold,
                             row = (b*Hq + h)*Sq + q_idx; fmix32 = MurmurHash3's
                             32-bit finalizer                                           */
    MM_MASK_DOCUMENT = 8u /* keep iff q_doc_ids[b][q_idx] == kv_doc_ids[b][kv_idx]: a
                             mask_mod that captures tensors (packed documents). The ids
                             must not decrease along the positions of a sequence (the
                             kernels skip whole tiles from the end ids); any int32
                             values, gaps allowed. Ids that do decrease give an
                             unspecified result, though every read stays within the
                             arrays. Composes with MM_MASK_CAUSAL, MM_MASK_WINDOW,
                             MM_MASK_ROWDROP and the block mask (inside partial
                             blocks). Forward and backward only (decode takes an
                             additive mask instead)                                     */
};

/*
 * Block mask (block sparsity, the phase FlyDSL PR #931 names as future work, in the
 * shape of PyTorch's BlockMask with its full and partial block lists): one byte per
 * (b, h, query block of MM_BLOCK_Q rows, key block of MM_BLOCK_KV keys):
 *   0        no pair of the block is kept; its keys are never read,
 *   1        partial: the mask_mod predicates (causal, window, document) decide per pair,
 *   2        full: every pair is kept and the predicates are not evaluated.
 * Other values are reserved and currently act as 2. MM_MASK_ROWDROP and the key-length
 * bound apply in every block. Byte (b, h, qb, kb) sits at
 *   block_mask[b*s[0] + h*s[1] + qb*s[2] + kb],  s = block_mask_strides,
 * for qb < ceil(Sq/MM_BLOCK_Q), kb < ceil(Skv/MM_BLOCK_KV); a stride of 0 broadcasts
 * that dimension. The table is a DEVICE pointer, borrowed like the tensors.
 */
#define MM_BLOCK_Q 128
#define MM_BLOCK_KV 64

typedef struct mm_mods {
    int32_t score_mod;            /* mm_score_mod                                      */
    uint32_t mask_flags;          /* OR of MM_MASK_*                                   */
    int32_t window;               /* MM_MASK_WINDOW half-width, 0..INT32_MAX; any value
                                     >= max(Sq, Skv) keeps every pair                   */
    uint32_t rowdrop_seed;        /* MM_MASK_ROWDROP                                   */
    uint32_t rowdrop_threshold;   /* MM_MASK_ROWDROP: ~threshold/2^32 of rows dropped  */
    const float *alibi_slopes;    /* device fp32 [Hq], or NULL for 2^(-8(h+1)/Hq)      */
    const uint8_t *block_mask;    /* device block mask (above), or NULL for none       */
    int64_t block_mask_strides[3];/* elements (bytes), for b, h, query block; >= 0     */
    const int32_t *q_doc_ids;     /* MM_MASK_DOCUMENT: device int32 [B, >= Sq], 4-byte
                                     aligned, contiguous along the sequence; required
                                     when B*Sq*Skv > 0 (MM_ERR_NULL), else unused       */
    const int32_t *kv_doc_ids;    /* MM_MASK_DOCUMENT: device int32 [B, >= Skv], same   */
    int64_t doc_strides[2];       /* elements between the sequences of q / kv ids, >= 0
                                     (MM_ERR_STRIDE); 0 shares one sequence's ids over
                                     the batch                                          */
} mm_mods;

typedef struct mm_fwd_args {
    const void *q;        /* [B, Hq, Sq, D]  dtype                                    */
    const void *k;        /* [B, Hkv, Skv, D] dtype                                   */
    const void *v;        /* [B, Hkv, Skv, D] dtype                                   */
    void *out;            /* [B, Hq, Sq, D]  dtype                                    */
    float *lse;           /* [B, Hq, Sq] fp32 contiguous, or NULL                     */
    int32_t dtype;        /* mm_dtype: MM_BF16, MM_F16, MM_FP8_E4M3 (MFMA paths) or
                             MM_F32; `out` has this dtype, except bf16 for fp8 inputs   */
    int32_t B, Hq, Hkv, Sq, Skv, D; /* D in {64, 128}; Sq, Skv < 2^30                 */
    int64_t q_strides[3]; /* elements, for b, h, s                                    */
    int64_t k_strides[3];
    int64_t v_strides[3];
    int64_t o_strides[3];
    float scale;          /* multiplies Q K^T before any mod                          */
    int32_t causal;       /* nonzero: same predicate as MM_MASK_CAUSAL                */
    mm_mods mods;
    /* MM_FP8_E4M3 only (ignored otherwise): per-tensor dequantisation factors, finite
     * and > 0. The attention is that of the real tensors descale_x * X8: the score is
     * scale * descale_q * descale_k * (Q8 . K8) and O is descale_v * softmax(...) V8.
     * The probabilities are rounded to e4m3 (round to nearest even) before the second
     * product and the row sum is taken over those rounded values; 16-byte aligned
     * bases and strides that are multiples of 16 elements are required. */
    float descale_q, descale_k, descale_v;
} mm_fwd_args;

typedef struct mm_decode_args {
    const void *q;           /* [B, Hq, 1, D] dtype                                   */
    const void *k_cache;     /* [B, Hkv, Scap, D] dtype                               */
    const void *v_cache;     /* [B, Hkv, Scap, D] dtype                               */
    void *out;               /* [B, Hq, 1, D] dtype                                   */
    float *lse;              /* [B, Hq] fp32 contiguous, or NULL                      */
    const void *mask;        /* f16 additive mask [B, Hq, 1, Scap] or NULL; added to
                                the scaled score; -inf masks a position              */
    const int32_t *seq_lens; /* device int32 [B] (each 0..kv_len), or NULL (= kv_len) */
    int32_t dtype;           /* MM_F16 or MM_BF16                                     */
    int32_t B, Hq, Hkv, kv_len, Scap, D; /* D in {64, 128}; 0 <= kv_len <= Scap        */
    float scale;             /* e.g. f16(1/sqrt(128)) = 0.08837890625                 */
    int64_t q_strides[2];    /* elements, for b, h                                    */
    int64_t kv_strides[3];   /* elements, for b, h, s (K and V share them)            */
    int64_t o_strides[2];    /* elements, for b, h                                    */
    int64_t mask_strides[2]; /* elements, for b, h (position stride is 1)             */
    void *workspace;         /* device scratch, >= mm_attn_decode_workspace_size()    */
    size_t workspace_bytes;
    int32_t num_splits;      /* 0 = automatic; else the KV split count to use         */
    /* Paged KV cache (the dynamic batch of the IREE issue with a page table): if
     * block_table is non-NULL, k_cache / v_cache are page pools [pages, Hkv, page_size,
     * D] with kv_strides = (page, head, row) strides, and position j of sequence b is row
     * j % page_size of page block_table[b * block_table_stride + j / page_size]. Entries
     * covering positions below the sequence's length must be valid page ids; no other
     * entry is read. page_size: a power of two. Scap is the logical capacity; with B > 1
 * the table's row stride must cover ceil(Scap / page_size) entries. */
    const int32_t *block_table;   /* device int32, or NULL for contiguous caches      */
    int64_t block_table_stride;   /* elements between sequences' rows of the table    */
    int32_t page_size;
} mm_decode_args;

typedef struct mm_bwd_args {
    const void *q, *k, *v;   /* the forward's inputs (as mm_fwd_args)                    */
    const void *out;         /* the forward's O [B, Hq, Sq, D]                           */
    const void *dout;        /* upstream gradient dO [B, Hq, Sq, D]                      */
    const float *lse;        /* the forward's LSE, fp32 contiguous [B, Hq, Sq] (required)*/
    void *dq;                /* [B, Hq, Sq, D]  outputs, dtype of the inputs             */
    void *dk;                /* [B, Hkv, Skv, D]                                         */
    void *dv;                /* [B, Hkv, Skv, D]                                         */
    int32_t dtype;           /* MM_BF16 or MM_F16                                         */
    int32_t B, Hq, Hkv, Sq, Skv, D; /* D in {64, 128}; Sq, Skv < 2^30                    */
    int64_t q_strides[3], k_strides[3], v_strides[3], o_strides[3], do_strides[3];
    int64_t dq_strides[3], dk_strides[3], dv_strides[3]; /* elements, for b, h, s        */
    float scale;             /* the forward's scale                                       */
    int32_t causal;          /* the forward's causal flag                                 */
    mm_mods mods;            /* the forward's mods (score_mod, mask_mods, block mask)     */
    void *workspace;         /* device scratch, >= mm_attn_bwd_workspace_size()           */
    size_t workspace_bytes;
} mm_bwd_args;

/* Forward attention. Returns MM_OK, or (launching nothing) MM_ERR_NULL for a missing
 * required pointer (q/out when B*Hq*Sq > 0, k/v when B*Hkv*Skv > 0, the document ids),
 * MM_ERR_DTYPE, MM_ERR_SHAPE (negative sizes, Sq or Skv >= 2^30, Hq % Hkv, window < 0,
 * non-finite scale or descales), MM_ERR_UNSUPPORTED (D, unknown score_mod or mask flag), MM_ERR_STRIDE
 * (negative strides, misaligned bases, strides that are not multiples of the vector
 * width, tiles whose byte offsets exceed 32 bits); MM_ERR_LAUNCH if the runtime reports
 * a launch failure. One launch on `stream`. */
mm_status mm_attn_fwd(const mm_fwd_args *args, void *stream);

/* Bytes of device workspace mm_attn_bwd needs (0 if invalid). */
size_t mm_attn_bwd_workspace_size(int32_t B, int32_t Hq, int32_t Sq);

/* Backward of mm_attn_fwd: the gradients of sum(dout * out) with respect to q, k and v,
 * for the same mods (the alibi bias, the mask_mods and the block mask do not depend on
 * q, k, v; masked pairs and rows with no kept key, LSE = -inf, contribute nothing;
 * with GQA the K/V gradients sum over the query heads of a group). Written from the
 * softmax Jacobian as in the FlyDSL PR's named future phase (backward): with
 * P = exp(s - LSE), dV = P^T dO, dS = P (dO V^T - rowsum(dO * O)), dQ = scale dS K,
 * dK = scale dS^T Q. P and dS are rounded to the input dtype for their products;
 * accumulation is fp32. Three launches on `stream` (a pre-pass into the workspace,
 * then dQ, then dK/dV); dq, dk, dv are written, not accumulated into. bf16/f16 only
 * (MM_ERR_DTYPE otherwise); a missing or short workspace gives MM_ERR_WORKSPACE; the
 * other checks are the forward's. */
mm_status mm_attn_bwd(const mm_bwd_args *args, void *stream);

/* Bytes of device workspace mm_attn_decode needs for these sizes (0 if invalid).
 * num_splits as in mm_decode_args (0 = automatic). Sized for the larger automatic
 * split count of a call with seq_lens, so it serves calls with and without them. */
size_t mm_attn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t kv_len, int32_t D,
                                     int32_t num_splits);

/* Decode attention (two launches on `stream`: split pass, then merge; one launch when
 * the split count is 1, the split pass then writing the output itself). With GQA
 * (Hq > Hkv) one workgroup of the split pass serves up to 4 query heads of a kv head,
 * so K/V are streamed once per 4 query heads (larger groups take several workgroups,
 * which the automatic split count places on one XCD so that they share its L2).
 * Rejections as for the forward, plus MM_ERR_SHAPE for kv_len > Scap or a bad page
 * size, MM_ERR_UNSUPPORTED for a split count outside 0..256 and MM_ERR_WORKSPACE for
 * a missing or short workspace. */
mm_status mm_attn_decode(const mm_decode_args *args, void *stream);

/* Bytes of the decode scratch that the library holds on each GPU for
 * mm_attn_decode_noalloc (16 MiB). */
#define MM_DECODE_SCRATCH_BYTES (16u * 1024u * 1024u)

/* Decode attention that allocates nothing and takes no workspace, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. The operation, kernels, split count and results are
 * those of mm_attn_decode with the same arguments; args->workspace and
 * args->workspace_bytes are ignored. The split partials (the B * Hq * splits * (D + 2)
 * floats that mm_attn_decode_workspace_size counts) go to a static device array of
 * MM_DECODE_SCRATCH_BYTES that the library holds on each GPU it runs on until the
 * process ends; its address is looked up once per device, on the first call with that
 * device current. No device memory is allocated or freed by any call.
 *   - A call whose partials need more than MM_DECODE_SCRATCH_BYTES returns
 *     MM_ERR_WORKSPACE and launches nothing (with the automatic split count that
 *     happens only beyond B * Hq = 32263 at D 128, 63550 at D 64).
 *   - `stream` must belong to the calling thread's current device; otherwise, or if the
 *     address lookup fails, the call returns MM_ERR_LAUNCH and launches nothing.
 *   - Every call on a GPU uses that GPU's one array, which keeps the last call's
 *     partials (each call writes every partial it reads, so nothing needs clearing).
 *     Calls that overlap in time on one GPU (on different streams, or from threads
 *     without ordering) race and give undefined results: order them, e.g. on one stream.
 * Other rejections as mm_attn_decode. Launches as mm_attn_decode. */
mm_status mm_attn_decode_noalloc(const mm_decode_args *args, void *stream);

/* Split count mm_attn_decode uses when num_splits == 0: about one resident round of
 * split workgroups (1024 with one query head per workgroup, 512 with 2 or 4), at least
 * 256 keys per split, at most 256 splits, a multiple of 8 (when 8 or more) if a kv
 * head's group spans several workgroups. Each split's key range is rounded up to a
 * whole number of the split loop's iterations, so the last splits of a row may be
 * empty (they contribute nothing; the workspace size does not change). */
int32_t mm_attn_decode_auto_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t kv_len);

/* Split count mm_attn_decode uses when num_splits == 0 and seq_lens is given. The
 * lengths are then known only on the device and one sequence may hold nearly all the
 * keys, so the count of mm_attn_decode_auto_splits is raised to the one a batch of a
 * single sequence would get, as far as the split workgroups stay within 8 resident
 * rounds (8192 with one query head per workgroup, 4096 with 2 or 4); the same bounds
 * and rounding apply. Splits past a sequence's length end at once and weigh nothing in
 * the merge. Equal to mm_attn_decode_auto_splits for B = 1. 0 if the sizes are invalid. */
int32_t mm_attn_decode_auto_splits_varlen(int32_t B, int32_t Hq, int32_t Hkv, int32_t kv_len);

/* Block-mask classes of the built-in mask_mods, the analogue of building a BlockMask
 * from a mask_mod: out[qb*ld + kb] (device bytes, qb < ceil(Sq/MM_BLOCK_Q),
 * kb < ceil(Skv/MM_BLOCK_KV), ld >= ceil(Skv/MM_BLOCK_KV)) gets 0 if the predicates of
 * `mask_flags` (MM_MASK_CAUSAL, MM_MASK_WINDOW with half-width `window`) keep no pair
 * (q_idx < Sq, kv_idx < Skv) of the block, 2 if they keep every such pair, else 1.
 * With no flag every block is 2. The table does not depend on b or h: pass it to
 * mm_attn_fwd with block_mask_strides {0, 0, ld} and the same mask_flags, and the
 * result equals that of the predicates alone, with empty blocks never read.
 * MM_MASK_ROWDROP and MM_MASK_DOCUMENT are rejected here (MM_ERR_UNSUPPORTED: the
 * first is per row, the second depends on the ids; mm_attn_fwd applies both anyway).
 * One launch on `stream`; Sq or Skv of 0 writes nothing. */
mm_status mm_block_mask_create(uint32_t mask_flags, int32_t window, int32_t Sq, int32_t Skv,
                               uint8_t *out, int64_t ld, void *stream);

/* Static string for a status code. */
const char *mm_status_str(int32_t status);

/* sizeof of the argument structs, for bindings to check their mirrored layout. */
size_t mm_fwd_args_size(void);
size_t mm_decode_args_size(void);
size_t mm_bwd_args_size(void);

/* Library version, major*10000 + minor*100 + patch. */
int32_t mm_version(void);

/* Identifier of the sources this library was compiled from (a hash of the kernel, ABI
 * and header files, "unknown" if the build did not set it). A binding can compare it
 * with the sources it ships to refuse a stale library. Static string, never freed. */
const char *mm_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* MASKMODS_H */
