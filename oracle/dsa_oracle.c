/*
 * dsa_oracle.c -- CPU oracle of the DSA sparse-attention step.
 *
 * TEST INFRASTRUCTURE ONLY (see dsa_oracle.h).  Plain loops, fp64, OpenMP
 * only across independent outputs.  No blocking, fusion or reordering beyond
 * what the definition states: scores are computed one position at a time,
 * selection is a full sort, attention is a two-pass softmax.
 */
#include "dsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------------------
 * Element decoding.
 *
 * bf16 is the upper half of an IEEE binary32 pattern.
 * e4m3 follows the OCP 8-bit floating point specification ("E4M3", the
 * variant with no infinities): 1 sign bit, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; the codes
 * with all exponent and mantissa bits set (0x7F, 0xFF) are NaN; the largest
 * finite magnitude is 1.75 * 2^8 = 448.  The FP8 storage itself is the
 * quantized route the pages name ("Optimizing Inference for Hybrid Attention
 * Architectures: From Operator Fusion to Sequence Sharding", section "Layered
 * Quantization: Distinguishing Precision Sensitivity").
 * ------------------------------------------------------------------------- */
double dsa_oracle_decode_bf16(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double dsa_oracle_decode_e4m3(uint8_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, -6);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return sign ? -v : v;
}

/* E8M0 (the shared scale of an OCP microscaling block): the byte is a
 * biased power-of-two exponent, value 2^(code - 127); code 255 is NaN. */
double dsa_oracle_decode_e8m0(uint8_t code)
{
    return code == 255 ? NAN : ldexp(1.0, (int)code - 127);
}

static double load_elem(const void *base, size_t i, int dtype)
{
    switch (dtype) {
    case 0: return (double)((const float *)base)[i];
    case 1: return dsa_oracle_decode_bf16(((const uint16_t *)base)[i]);
    case 2:
    case 3: return dsa_oracle_decode_e4m3(((const uint8_t *)base)[i]);
    default: return NAN;
    }
}

/* Scale of element d of a stored vector (row `r` of a scale array): fp8 one
 * fp32 scale per vector, MXFP8 one E8M0 byte per 32 elements, else 1. */
static double elem_scale(const void *scale, size_t r, int D, int d, int dtype)
{
    if (dtype == 2)
        return (double)((const float *)scale)[r];
    if (dtype == 3)
        return dsa_oracle_decode_e8m0(((const uint8_t *)scale)[r * (size_t)(D / 32) + d / 32]);
    return 1.0;
}

static int set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0)
        omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    return 0;
}

/* Request that owns query row i (rows of request b are
 * [q_offsets[b], q_offsets[b+1])). */
static int request_of_row(int B, const int32_t *q_offsets, int i)
{
    for (int b = 0; b < B; ++b)
        if (i >= q_offsets[b] && i < q_offsets[b + 1])
            return b;
    return -1;
}

/* Causal visibility.  A request's cached positions include its own query
 * tokens, so its n_b query rows are its last n_b positions; row j may see the
 * positions up to and including its own.  The pages state the causal rule for
 * the index computation ("Day0 Inference Support and Performance Optimization
 * for New LLM Architectures", section V, 5.2: later tokens see a longer
 * history). */
int dsa_oracle_visible(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                       int32_t *vis)
{
    if (B < 0 || !q_offsets || !ctx_lens || !vis)
        return -1;
    for (int b = 0; b < B; ++b) {
        int n = q_offsets[b + 1] - q_offsets[b];
        if (n < 0 || ctx_lens[b] < n)
            return -2;
        for (int j = 0; j < n; ++j)
            vis[q_offsets[b] + j] = ctx_lens[b] - n + j + 1;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Lightning-indexer scores.
 *
 * Phase 1 of the DSA step scores the relevance of every historical position
 * to the current query and weights the per-head scores by head importance
 * ("Optimizing Inference for Hybrid Attention Architectures: From Operator
 * Fusion to Sequence Sharding", section "Breaking Down the Computational Path
 * of Hybrid Attention", item 1).  The form used is
 *     s_t = sum_h w_h * max(sum_d q[h][d] * k_t[d], 0),
 * one key row k_t per position shared by all indexer heads.  Keys are read
 * from the paged K cache through the block table ("Day0 Inference Support and
 * Performance Optimization for New LLM Architectures", section III, 3.1).
 * For the fp8 route each stored value is code * scale, with one scale per
 * (query row, head) for q and one per cached token for k.  The MXFP8 route
 * (q and k quantized in groups of 32 elements that share one scale: "Optimizing
 * Inference for Hybrid Attention Architectures: From Operator Fusion to
 * Sequence Sharding", section "Layered Quantization: Distinguishing Precision
 * Sensitivity"; "Day0 Inference Optimization for Next-Generation
 * Hybrid-Architecture LLMs Based on CANN", section 3.1) stores e4m3 codes and
 * one E8M0 byte per 32 consecutive elements of each q and k vector; each
 * stored value is code * 2^(E - 127).
 * ------------------------------------------------------------------------- */
int dsa_oracle_scores(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                      const int32_t *block_table, int bt_stride, int page_size,
                      int H, int D, int dtype,
                      const void *q, const void *q_scale, const float *w,
                      const void *k_cache, const void *k_scale,
                      int L_out, double *scores, int nthreads)
{
    if (B < 0 || H <= 0 || D <= 0 || page_size <= 0 || L_out < 0 || !q_offsets ||
        !ctx_lens || !block_table || !q || !w || !k_cache || !scores)
        return -1;
    if (dtype < 0 || dtype > 3)
        return -1;
    if (dtype >= 2 && (!q_scale || !k_scale))
        return -1;
    if (dtype == 3 && D % 32 != 0)
        return -1;
    int T = q_offsets[B];
    int32_t *vis = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    if (!vis)
        return -3;
    if (dsa_oracle_visible(B, q_offsets, ctx_lens, vis)) {
        free(vis);
        return -2;
    }
    for (int i = 0; i < T; ++i)
        if (vis[i] > L_out) {
            free(vis);
            return -2;
        }
    set_threads(nthreads);

    for (int i = 0; i < T; ++i) {
        int b = request_of_row(B, q_offsets, i);
        /* decode this row's query and weights once */
        double *qd = (double *)malloc(sizeof(double) * (size_t)H * D);
        double *wd = (double *)malloc(sizeof(double) * (size_t)H);
        for (int h = 0; h < H; ++h) {
            for (int d = 0; d < D; ++d)
                qd[(size_t)h * D + d] = load_elem(q, ((size_t)i * H + h) * D + d, dtype) *
                                        elem_scale(q_scale, (size_t)i * H + h, D, d, dtype);
            wd[h] = (double)w[(size_t)i * H + h];
        }
        double *row = scores + (size_t)i * L_out;
        int n_vis = vis[i];
#pragma omp parallel for schedule(static)
        for (int t = 0; t < L_out; ++t) {
            if (t >= n_vis) {
                row[t] = NAN;
                continue;
            }
            int page = block_table[(size_t)b * bt_stride + t / page_size];
            int slot = t % page_size;
            size_t tok = (size_t)page * page_size + slot;
            size_t base = tok * D;
            double s = 0.0;
            for (int h = 0; h < H; ++h) {
                double logit = 0.0;
                for (int d = 0; d < D; ++d)
                    logit += qd[(size_t)h * D + d] *
                             (load_elem(k_cache, base + d, dtype) * elem_scale(k_scale, tok, D, d, dtype));
                s += wd[h] * (logit > 0.0 ? logit : 0.0);
            }
            row[t] = s;
        }
        free(qd);
        free(wd);
    }
    free(vis);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Top-K selection.
 *
 * The Top-K historical positions become the sparse index set ("Optimizing
 * Inference for Hybrid Attention Architectures: From Operator Fusion to
 * Sequence Sharding", section "Breaking Down the Computational Path of Hybrid
 * Attention", item 1).  Reading adopted: order positions by score descending
 * and, among equal scores, by position ascending (numeric comparison, so -0
 * and +0 are equal); keep the first min(K, visible); write the kept positions
 * in ascending order (the "index rearrangement" of "Optimizing Inference for
 * Hybrid Attention LLMs: Practices for Fast Adaptation", section 3, item 2);
 * pad with -1.
 * ------------------------------------------------------------------------- */
typedef struct {
    double s;
    int32_t t;
} scored_pos;

static int by_score_then_position(const void *a, const void *b)
{
    const scored_pos *x = (const scored_pos *)a, *y = (const scored_pos *)b;
    if (x->s > y->s) return -1;
    if (x->s < y->s) return 1;
    return (x->t > y->t) - (x->t < y->t);
}

static int ascending_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

int dsa_oracle_select(int T, int L_out, const double *scores, const int32_t *vis,
                      int K, int32_t *idx, int nthreads)
{
    if (T < 0 || L_out < 0 || K <= 0 || !scores || !vis || !idx)
        return -1;
    for (int i = 0; i < T; ++i)
        if (vis[i] < 0 || vis[i] > L_out)
            return -2;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int i = 0; i < T; ++i) {
        int n = vis[i];
        scored_pos *all = (scored_pos *)malloc(sizeof(scored_pos) * (size_t)(n > 0 ? n : 1));
        for (int t = 0; t < n; ++t) {
            all[t].s = scores[(size_t)i * L_out + t];
            all[t].t = t;
        }
        qsort(all, (size_t)n, sizeof(scored_pos), by_score_then_position);
        int keep = n < K ? n : K;
        int32_t *out = idx + (size_t)i * K;
        for (int r = 0; r < keep; ++r)
            out[r] = all[r].t;
        qsort(out, (size_t)keep, sizeof(int32_t), ascending_i32);
        for (int r = keep; r < K; ++r)
            out[r] = -1;
        free(all);
    }
    return 0;
}

int dsa_oracle_indexer_topk(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                            const int32_t *block_table, int bt_stride, int page_size,
                            int H, int D, int dtype,
                            const void *q, const void *q_scale, const float *w,
                            const void *k_cache, const void *k_scale,
                            int K, int32_t *idx, int L_out, double *scores_out,
                            int nthreads)
{
    if (B < 0 || !q_offsets || !ctx_lens || K <= 0 || !idx)
        return -1;
    int T = q_offsets[B];
    double *scores = scores_out;
    if (!scores) {
        scores = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * (size_t)(L_out > 0 ? L_out : 1));
        if (!scores)
            return -3;
    }
    int32_t *vis = (int32_t *)malloc(sizeof(int32_t) * (size_t)(T > 0 ? T : 1));
    int rc = dsa_oracle_visible(B, q_offsets, ctx_lens, vis);
    if (!rc)
        rc = dsa_oracle_scores(B, q_offsets, ctx_lens, block_table, bt_stride, page_size, H, D,
                               dtype, q, q_scale, w, k_cache, k_scale, L_out, scores, nthreads);
    if (!rc)
        rc = dsa_oracle_select(T, L_out, scores, vis, K, idx, nthreads);
    free(vis);
    if (scores != scores_out)
        free(scores);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Sparse attention over the selected positions.
 *
 * Phase 2 of the DSA step reads the cached entries of the selected positions
 * only and attends over them ("Optimizing Inference for Hybrid Attention
 * Architectures: From Operator Fusion to Sequence Sharding", section
 * "Breaking Down the Computational Path of Hybrid Attention", item 2; "Day0
 * Inference Support and Performance Optimization for New LLM Architectures",
 * section III, 3.2).  The cache is the latent cache of multi-head latent
 * attention: one shared row c_t per position, used whole as the key and by
 * its first Dv entries as the value.  For each query row i and head h:
 *     z_t = scale * (q[i][h] . c_t)          over the selected t
 *     m = max z,  l = sum_t exp(z_t - m)
 *     out[i][h][e] = sum_t exp(z_t - m) * c_t[e] / l,   lse = m + ln l.
 * ------------------------------------------------------------------------- */
int dsa_oracle_sparse_attn(int B, const int32_t *q_offsets,
                           const int32_t *block_table, int bt_stride, int page_size,
                           int H, int Dqk, int Dv, int dtype, double scale,
                           const void *q, const void *kv_cache,
                           const int32_t *idx, int K,
                           double *out, double *lse, int nthreads)
{
    if (B < 0 || !q_offsets || !block_table || H <= 0 || Dqk <= 0 || Dv <= 0 || Dv > Dqk ||
        page_size <= 0 || !q || !kv_cache || !idx || K <= 0 || !out)
        return -1;
    if (dtype != 0 && dtype != 1)
        return -1;
    int T = q_offsets[B];
    set_threads(nthreads);
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int i = 0; i < T; ++i) {
        for (int h = 0; h < H; ++h) {
            int b = request_of_row(B, q_offsets, i);
            const int32_t *sel = idx + (size_t)i * K;
            double *z = (double *)malloc(sizeof(double) * (size_t)K);
            double *qd = (double *)malloc(sizeof(double) * (size_t)Dqk);
            for (int d = 0; d < Dqk; ++d)
                qd[d] = load_elem(q, ((size_t)i * H + h) * Dqk + d, dtype);
            double m = -INFINITY;
            for (int r = 0; r < K; ++r) {
                int t = sel[r];
                if (t < 0)
                    continue;
                int page = block_table[(size_t)b * bt_stride + t / page_size];
                size_t base = ((size_t)page * page_size + t % page_size) * Dqk;
                double dot = 0.0;
                for (int d = 0; d < Dqk; ++d)
                    dot += qd[d] * load_elem(kv_cache, base + d, dtype);
                z[r] = scale * dot;
                if (z[r] > m)
                    m = z[r];
            }
            double *o = out + ((size_t)i * H + h) * Dv;
            for (int e = 0; e < Dv; ++e)
                o[e] = 0.0;
            double l = 0.0;
            for (int r = 0; r < K; ++r) {
                int t = sel[r];
                if (t < 0)
                    continue;
                double p = exp(z[r] - m);
                l += p;
                int page = block_table[(size_t)b * bt_stride + t / page_size];
                size_t base = ((size_t)page * page_size + t % page_size) * Dqk;
                for (int e = 0; e < Dv; ++e)
                    o[e] += p * load_elem(kv_cache, base + e, dtype);
            }
            if (l > 0.0) {
                for (int e = 0; e < Dv; ++e)
                    o[e] /= l;
                if (lse)
                    lse[(size_t)i * H + h] = m + log(l);
            } else if (lse) {
                lse[(size_t)i * H + h] = -INFINITY;
            }
            free(z);
            free(qd);
        }
    }
    return 0;
}
