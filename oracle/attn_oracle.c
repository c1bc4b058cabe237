/*
 * attn_oracle.c -- the oracle: a plain, slow CPU attention in float64.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product (the HIP library and its
 * Python binding) never calls it and shares no code with it.
 *
 * What it computes (flex_attention semantics as described on the pages):
 *   For each batch b, query head h, query row i, with kv head hk = h / (Hq/Hkv)
 *   (GQA groups of consecutive query heads share one K/V head -- the
 *   enable_gqa operand of the torch-mlir flex_attention op, PR #4366 description):
 *     s_j  = scale * sum_d Q[b,h,i,d] * K[b,hk,j,d]               (fp64)
 *     s_j += slope_h * (j - i)           if the alibi score_mod is on; the mod
 *                                        sees the already-scaled score
 *                                        ("scale-then-mod", FlyDSL PR #931, Summary)
 *     s_j += mask[b,h,i,j]               if an additive mask is given (decode
 *                                        form of IREE issue #19015: the mask is an
 *                                        operand of the attention op next to Q,K,V
 *                                        and the scale, added to the scaled score)
 *     kept_j = mask_mod(b,h,i,j) AND j < len_b ; s_j = -inf if not kept
 *                                        (mask applied after the score_mod,
 *                                        FlyDSL PR #931, Summary)
 *   If no key is kept (or every kept s_j is -inf): O = 0, LSE = -inf
 *   (the fully-masked-row guard, FlyDSL PR #931, Summary). Otherwise
 *     M = max_j s_j,  w_j = exp(s_j - M),  Lsum = sum_j w_j,
 *     O[b,h,i,:] = sum_j w_j V[b,hk,j,:] / Lsum,   LSE = M + ln(Lsum).
 *
 * mask_mod predicates (true = keep), AND-composed:
 *   causal:          j <= i          (raw indices, top-left aligned when Sq != Skv)
 *   sliding window:  |i - j| <= w    (inclusive; the pages' built-in pairs it with causal)
 *   row drop:        fmix32(seed ^ ((b*Hq + h)*Sq + i)) >= threshold, else the
 *                    whole row is masked. fmix32 is the 32-bit finalizer of
 *                    Austin Appleby's MurmurHash3 (public domain).
 * alibi slope for query head h of H: 2^(-8(h+1)/H) unless slopes are given.
 *
 * Document mask (optional, a mask_mod that captures tensors): keep iff
 * q_doc[b][i] == kv_doc[b][j], AND-composed with the other predicates.
 *
 * Block mask (optional, BlockMask-style): one byte per (b, h, q block of 128 rows,
 * kv block of 64 keys): 0 = no pair of the block is kept; 2 = every pair is kept and
 * the mask_mod predicates (causal, window) are not evaluated there; 1 = the predicates
 * decide. The row-drop mod and the key-length bound apply everywhere. This is the
 * FlyDSL PR's named future phase (block sparsity), read as PyTorch's BlockMask with
 * its full / partial block lists.
 *
 * Backward (oracle_attention_bwd): the gradients of sum(dO * O) with respect to q, k, v
 * written out from the softmax Jacobian, over the same scores (below).
 *
 * Inputs are float64 arrays holding the exact values of the bf16/f16/f32 inputs.
 * Nothing here is blocked, fused, reordered or rounded beyond that definition.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

uint32_t oracle_fmix32(uint32_t h)
{
    h ^= h >> 16;
    h *= 0x85ebca6bu;
    h ^= h >> 13;
    h *= 0xc2b2ae35u;
    h ^= h >> 16;
    return h;
}

int oracle_row_dropped(uint32_t seed, uint32_t threshold, int64_t row)
{
    return oracle_fmix32(seed ^ (uint32_t)row) < threshold;
}

double oracle_alibi_slope(int h, int H)
{
    return pow(2.0, -8.0 * (double)(h + 1) / (double)H);
}

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

typedef struct {
    int B, Hq, Hkv, Sq, Skv, D, kv_cap;
    const double *q, *k, *v;
    double scale;
    int alibi;
    const double *slopes;
    int causal, window, rowdrop;
    uint32_t seed, threshold;
    const double *add_mask;
    int64_t mask_ld;
    const int32_t *lens;
    const uint8_t *block_mask;
    int64_t bm_sb, bm_sh, bm_sq;
    const int32_t *q_doc, *kv_doc;  /* document ids per position, or NULL */
    int64_t q_doc_sb, kv_doc_sb;
} problem;

#define ORACLE_BLOCK_Q 128
#define ORACLE_BLOCK_KV 64

/* The final scores of one query row: s[j] = scale*q.k (+ alibi) (+ additive mask), or
 * -inf where the mask_mods / block mask / length drop the pair. Returns their max. */
static double row_scores(const problem *p, int b, int h, int i, double *s)
{
    const int group = p->Hq / p->Hkv;
    const int hk = h / group;
    const int64_t row = ((int64_t)b * p->Hq + h) * p->Sq + i;
    const double *qi = p->q + row * p->D;
    const double *kb = p->k + ((int64_t)b * p->Hkv + hk) * p->kv_cap * p->D;
    const int len = p->lens ? p->lens[b] : p->Skv;
    const int dropped = p->rowdrop && oracle_row_dropped(p->seed, p->threshold, row);
    const double slope = p->alibi ? (p->slopes ? p->slopes[h] : oracle_alibi_slope(h, p->Hq)) : 0.0;

    double M = -INFINITY;
    for (int j = 0; j < p->Skv; ++j) {
        int keep = !dropped && j < len;
        int blk = 1;
        if (p->block_mask)
            blk = p->block_mask[b * p->bm_sb + h * p->bm_sh + (int64_t)(i / ORACLE_BLOCK_Q) * p->bm_sq +
                                j / ORACLE_BLOCK_KV];
        if (blk == 0) keep = 0;
        if (blk == 1) {
            if (p->causal && !(j <= i)) keep = 0;
            if (p->window >= 0 && !(abs(i - j) <= p->window)) keep = 0;
            if (p->q_doc && p->q_doc[b * p->q_doc_sb + i] != p->kv_doc[b * p->kv_doc_sb + j]) keep = 0;
        }
        if (!keep) {
            s[j] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int d = 0; d < p->D; ++d) dot += qi[d] * kb[(int64_t)j * p->D + d];
        double x = p->scale * dot;
        if (p->alibi) x += slope * (double)(j - i);
        if (p->add_mask) x += p->add_mask[row * p->mask_ld + j];
        s[j] = x;
        if (x > M) M = x;
    }
    return M;
}

/* One query row. s: scratch of Skv doubles. o: D outputs. wsq, wvar: NULL or the
 * row's first-order sensitivity to relative perturbations of the weights (below). */
static void attend_row(const problem *p, int b, int h, int i, double *s, double *o, double *lse,
                       double *wsq, double *wvar)
{
    const int hk = h / (p->Hq / p->Hkv);
    const double *vb = p->v + ((int64_t)b * p->Hkv + hk) * p->kv_cap * p->D;
    const double M = row_scores(p, b, h, i, s);
    for (int d = 0; d < p->D; ++d) o[d] = 0.0;
    if (wsq) *wsq = 0.0;
    if (wvar)
        for (int d = 0; d < p->D; ++d) wvar[d] = 0.0;
    if (M == -INFINITY) {
        *lse = -INFINITY;
        return;
    }
    double Lsum = 0.0;
    for (int j = 0; j < p->Skv; ++j) {
        if (s[j] == -INFINITY) continue;
        double w = exp(s[j] - M);
        Lsum += w;
        for (int d = 0; d < p->D; ++d) o[d] += w * vb[(int64_t)j * p->D + d];
    }
    for (int d = 0; d < p->D; ++d) o[d] /= Lsum;
    *lse = M + log(Lsum);
    if (!wsq && !wvar) return;
    /* w_j = exp(s_j - M) / Lsum; if every weight is perturbed to w_j (1 + e_j) (and the
     * weights renormalised), O_d moves by sum_j e_j w_j (v_jd - O_d) and LSE by
     * sum_j e_j w_j, to first order. With independent e_j of variance t^2 their standard
     * deviations are t * sqrt(wvar_d) and t * sqrt(wsq). */
    for (int j = 0; j < p->Skv; ++j) {
        if (s[j] == -INFINITY) continue;
        const double w = exp(s[j] - M) / Lsum;
        if (wsq) *wsq += w * w;
        if (wvar)
            for (int d = 0; d < p->D; ++d) {
                const double dv = vb[(int64_t)j * p->D + d] - o[d];
                wvar[d] += w * w * dv * dv;
            }
    }
}

/*
 * Returns 0 on success, -1 on invalid arguments.
 *   q      [B,Hq,Sq,D]        contiguous
 *   k, v   [B,Hkv,kv_cap,D]   contiguous; keys 0..Skv-1 are used (Skv <= kv_cap)
 *   window < 0 disables the sliding window
 *   add_mask: NULL or additive bias, element (row, j) at add_mask[row*mask_ld + j]
 *   lens:  NULL or per-batch key count (keys j >= lens[b] are masked)
 *   block_mask: NULL or bytes indexed b*bm_sb + h*bm_sh + (i/128)*bm_sq + j/64
 *   rows:  NULL -> every row in order; else nrows flat row ids (b*Hq + h)*Sq + i
 *   out [nrows, D], lse [nrows]
 *   wsq [nrows], wvar [nrows, D]: NULL, or per row sum_j w_j^2 and per element
 *          sum_j w_j^2 (V[j,d] - O[d])^2 over the kept keys (w_j the softmax weights):
 *          the first-order scale of the LSE and O errors that independent relative
 *          errors in the weights cause (used to size the fp8 tolerance)
 */
int oracle_attention(int B, int Hq, int Hkv, int Sq, int Skv, int D,
                     const double *q, const double *k, const double *v, int kv_cap,
                     double scale, int alibi, const double *slopes,
                     int causal, int window, int rowdrop, uint32_t seed, uint32_t threshold,
                     const double *add_mask, int64_t mask_ld, const int32_t *lens,
                     const uint8_t *block_mask, int64_t bm_sb, int64_t bm_sh, int64_t bm_sq,
                     const int32_t *q_doc, const int32_t *kv_doc, int64_t q_doc_sb, int64_t kv_doc_sb,
                     const int64_t *rows, int64_t nrows, double *out, double *lse,
                     double *wsq, double *wvar)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0) return -1;
    if (Hq % Hkv != 0 || kv_cap < Skv) return -1;
    if (!q || !k || !v || !out || !lse) return -1;
    const int64_t total = (int64_t)B * Hq * Sq;
    if (!rows) nrows = total;
    if ((q_doc == NULL) != (kv_doc == NULL)) return -1;
    problem p = {B, Hq, Hkv, Sq, Skv, D, kv_cap, q, k, v, scale, alibi, slopes,
                 causal, window, rowdrop, seed, threshold, add_mask, mask_ld, lens,
                 block_mask, bm_sb, bm_sh, bm_sq, q_doc, kv_doc, q_doc_sb, kv_doc_sb};
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        if (!s) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 4)
            for (int64_t n = 0; n < nrows; ++n) {
                const int64_t r = rows ? rows[n] : n;
                if (r < 0 || r >= total) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                const int i = (int)(r % Sq);
                const int h = (int)((r / Sq) % Hq);
                const int b = (int)(r / ((int64_t)Sq * Hq));
                attend_row(&p, b, h, i, s, out + n * D, lse + n, wsq ? wsq + n : NULL,
                           wvar ? wvar + n * D : NULL);
            }
        }
        free(s);
    }
    return bad ? -1 : 0;
}

/*
 * Gradients of the forward above (no additive mask, no lengths) with respect to q, k, v
 * for an upstream gradient dO, from the definition: with P_ij = exp(s_ij - LSE_i) over
 * the kept pairs and O_i = sum_j P_ij V_j,
 *   dV_j = sum_i P_ij dO_i
 *   dP_ij = dO_i . V_j,   D_i = dO_i . O_i = sum_j P_ij dP_ij
 *   dS_ij = P_ij (dP_ij - D_i)                (softmax Jacobian)
 *   dQ_i = scale * sum_j dS_ij K_j,  dK_j = scale * sum_i dS_ij Q_i
 * The alibi bias and the masks do not depend on q, k, v: masked pairs have P = 0 and
 * contribute nothing; fully masked (and dropped) rows give zero gradients. With GQA the
 * K/V gradients of a kv head sum over the query heads that read it.
 * Layouts as oracle_attention (k, v, dk, dv with kv_cap = Skv). Parallel over (b, kv
 * head), so each K/V gradient has one writer. Returns 0, or -1 on invalid arguments.
 */
int oracle_attention_bwd(int B, int Hq, int Hkv, int Sq, int Skv, int D,
                         const double *q, const double *k, const double *v, const double *dout,
                         double scale, int alibi, const double *slopes,
                         int causal, int window, int rowdrop, uint32_t seed, uint32_t threshold,
                         const uint8_t *block_mask, int64_t bm_sb, int64_t bm_sh, int64_t bm_sq,
                         const int32_t *q_doc, const int32_t *kv_doc, int64_t q_doc_sb, int64_t kv_doc_sb,
                         double *dq, double *dk, double *dv)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Sq < 0 || Skv < 0 || D <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (!q || !k || !v || !dout || !dq || !dk || !dv) return -1;
    if ((q_doc == NULL) != (kv_doc == NULL)) return -1;
    problem p = {B, Hq, Hkv, Sq, Skv, D, Skv, q, k, v, scale, alibi, slopes,
                 causal, window, rowdrop, seed, threshold, NULL, 0, NULL,
                 block_mask, bm_sb, bm_sh, bm_sq, q_doc, kv_doc, q_doc_sb, kv_doc_sb};
    const int group = Hq / Hkv;
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        double *o = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !o) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bk = 0; bk < (int64_t)B * Hkv; ++bk) {
                const int b = (int)(bk / Hkv), hk = (int)(bk % Hkv);
                const double *kb = k + bk * Skv * D, *vb = v + bk * Skv * D;
                double *dkb = dk + bk * Skv * D, *dvb = dv + bk * Skv * D;
                for (int64_t t = 0; t < (int64_t)Skv * D; ++t) dkb[t] = dvb[t] = 0.0;
                for (int h = hk * group; h < (hk + 1) * group; ++h) {
                    for (int i = 0; i < Sq; ++i) {
                        const int64_t row = ((int64_t)b * Hq + h) * Sq + i;
                        const double *qi = q + row * D, *doi = dout + row * D;
                        double *dqi = dq + row * D;
                        for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                        const double M = row_scores(&p, b, h, i, s);
                        if (M == -INFINITY) continue;
                        double Lsum = 0.0;
                        for (int j = 0; j < Skv; ++j)
                            if (s[j] != -INFINITY) Lsum += exp(s[j] - M);
                        const double lse = M + log(Lsum);
                        /* O_i and D_i */
                        for (int d = 0; d < D; ++d) o[d] = 0.0;
                        for (int j = 0; j < Skv; ++j) {
                            if (s[j] == -INFINITY) continue;
                            const double pij = exp(s[j] - lse);
                            for (int d = 0; d < D; ++d) o[d] += pij * vb[(int64_t)j * D + d];
                        }
                        double Di = 0.0;
                        for (int d = 0; d < D; ++d) Di += doi[d] * o[d];
                        for (int j = 0; j < Skv; ++j) {
                            if (s[j] == -INFINITY) continue;
                            const double pij = exp(s[j] - lse);
                            double dpij = 0.0;
                            for (int d = 0; d < D; ++d) dpij += doi[d] * vb[(int64_t)j * D + d];
                            const double dsij = pij * (dpij - Di);
                            for (int d = 0; d < D; ++d) {
                                dvb[(int64_t)j * D + d] += pij * doi[d];
                                dqi[d] += scale * dsij * kb[(int64_t)j * D + d];
                                dkb[(int64_t)j * D + d] += scale * dsij * qi[d];
                            }
                        }
                    }
                }
            }
        }
        free(s);
        free(o);
    }
    return bad ? -1 : 0;
}
