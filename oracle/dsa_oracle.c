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
/* Element d of latent row `row` (pool row: page * page_size + slot).  fp32
 * and bf16 rows hold Dqk elements.  The fp8 latent row (dtype 2; "Day0
 * Inference Optimization for Next-Generation Hybrid-Architecture LLMs Based
 * on CANN", section 3.2, and "Optimizing Inference for Hybrid Attention
 * Architectures: From Operator Fusion to Sequence Sharding", section
 * "Layered Quantization: Distinguishing Precision Sensitivity": an fp8 KV
 * cache with one scale per token and 128-element tile) is Dv e4m3 codes, then
 * a 16-byte block holding Dv/128 E8M0 scale bytes (tile j covers codes
 * 128j .. 128j + 127; the rest of the block is unused), then the Dqk - Dv
 * rope elements in bf16: Dv + 16 + 2 (Dqk - Dv) bytes. */
static double latent_elem(const void *kv, size_t row, int d, int Dqk, int Dv, int dtype)
{
    if (dtype != 2)
        return load_elem(kv, row * Dqk + d, dtype);
    size_t row_bytes = (size_t)Dv + 16 + 2 * (size_t)(Dqk - Dv);
    const unsigned char *r = (const unsigned char *)kv + row * row_bytes;
    if (d < Dv)
        return dsa_oracle_decode_e4m3(r[d]) * dsa_oracle_decode_e8m0(r[Dv + d / 128]);
    uint16_t bits;
    memcpy(&bits, r + Dv + 16 + 2 * (d - Dv), sizeof bits);
    return dsa_oracle_decode_bf16(bits);
}

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
    if (dtype != 0 && dtype != 1 && dtype != 2)
        return -1;
    if (dtype == 2 && (Dv % 128 != 0 || Dv / 128 > 16))
        return -1;
    int q_dtype = dtype == 2 ? 1 : dtype; /* the fp8 latent route takes bf16 queries */
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
                qd[d] = load_elem(q, ((size_t)i * H + h) * Dqk + d, q_dtype);
            double m = -INFINITY;
            for (int r = 0; r < K; ++r) {
                int t = sel[r];
                if (t < 0)
                    continue;
                int page = block_table[(size_t)b * bt_stride + t / page_size];
                size_t prow = (size_t)page * page_size + t % page_size;
                double dot = 0.0;
                for (int d = 0; d < Dqk; ++d)
                    dot += qd[d] * latent_elem(kv_cache, prow, d, Dqk, Dv, dtype);
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
                size_t prow = (size_t)page * page_size + t % page_size;
                for (int e = 0; e < Dv; ++e)
                    o[e] += p * latent_elem(kv_cache, prow, e, Dqk, Dv, dtype);
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

/* ---- Cache append: the producer step that fills the indexer K pool --------
 * ("Optimizing Inference for Hybrid Attention Architectures: From Operator
 * Fusion to Sequence Sharding", section "Breaking Down the Computational Path
 * of Hybrid Attention": the normalised key of each new token is written into
 * the indexer's paged K cache, quantised where the indexer runs in low
 * precision; section "Layered Quantization: Distinguishing Precision
 * Sensitivity" for the MXFP8 grouping.)
 *
 * Placement: the n_b new keys of request b are its query tokens, so key j goes
 * to position p = L_b - n_b + j (where the scoring looks for it): page
 * block_table[b][p / page_size], slot p % page_size.
 *
 * Rounding: the codes are integer decisions taken from fp32 values, so the
 * quotients are formed in fp32 and rounded from there to the storage grid,
 * to nearest with ties to even.  round_to_grid is that rounding for a format
 * with `mant` fraction bits whose exponent stops at `emin` (below 2^emin the
 * spacing stays 2^(emin - mant): the subnormals). */
static double round_to_grid(double a, int mant, int emin)
{
    if (a == 0.0)
        return 0.0;
    int e;
    frexp(a, &e); /* a = f * 2^e with f in [0.5, 1), so floor(log2 a) = e - 1 */
    int E = e - 1 < emin ? emin : e - 1;
    double q = ldexp(1.0, E - mant);
    return nearbyint(a / q) * q; /* the default rounding mode: ties to even */
}

/* e4m3 code of v: nearest even, saturating at +-448, sign kept on zero. */
static uint8_t e4m3_of(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double r = round_to_grid(fabs(v), 3, -6);
    if (r > 448.0)
        r = 448.0;
    if (r == 0.0)
        return sign;
    int e;
    frexp(r, &e);
    int E = e - 1;
    if (E < -6) /* subnormal: a multiple of 2^-9 below 2^-6 */
        return (uint8_t)(sign | (int)(r / ldexp(1.0, -9)));
    return (uint8_t)(sign | ((E + 7) << 3) | (int)(r / ldexp(1.0, E - 3) - 8.0));
}

uint8_t dsa_oracle_encode_e4m3(float x)
{
    return e4m3_of((double)x);
}

uint16_t dsa_oracle_encode_bf16(float x)
{
    double r = round_to_grid(fabs((double)x), 7, -126);
    float f = (float)(signbit(x) ? -r : r); /* exact: r has at most 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

int dsa_oracle_cache_append(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                            const int32_t *block_table, int bt_stride, int page_size, int D,
                            int src_dtype, const void *k_new, int dst_dtype,
                            void *k_cache, void *k_scale)
{
    if (B < 1 || D < 1 || page_size < 1 || !q_offsets || !ctx_lens || !block_table || !k_new || !k_cache)
        return -1;
    if ((src_dtype != 0 && src_dtype != 1) || dst_dtype < 0 || dst_dtype > 3)
        return -1;
    if ((dst_dtype == 2 || dst_dtype == 3) && !k_scale)
        return -1;
    if (dst_dtype == 3 && D % 32 != 0)
        return -1;
    float *x = malloc(sizeof(float) * (size_t)D);
    if (!x)
        return -2;
    for (int b = 0; b < B; ++b) {
        int n = q_offsets[b + 1] - q_offsets[b], L = ctx_lens[b];
        if (n < 0 || n > L) {
            free(x);
            return -1;
        }
        for (int j = 0; j < n; ++j) {
            size_t i = (size_t)q_offsets[b] + j;
            int p = L - n + j;
            int page = block_table[(size_t)b * bt_stride + p / page_size];
            size_t row = (size_t)page * page_size + p % page_size;
            for (int d = 0; d < D; ++d)
                x[d] = (float)load_elem(k_new, i * D + d, src_dtype); /* exact */
            if (dst_dtype == 0) {
                for (int d = 0; d < D; ++d)
                    ((float *)k_cache)[row * D + d] = x[d];
            } else if (dst_dtype == 1) {
                for (int d = 0; d < D; ++d)
                    ((uint16_t *)k_cache)[row * D + d] = dsa_oracle_encode_bf16(x[d]);
            } else if (dst_dtype == 2) {
                float amax = 0.0f;
                for (int d = 0; d < D; ++d)
                    amax = fabsf(x[d]) > amax ? fabsf(x[d]) : amax;
                float s = amax > 0.0f ? amax / 448.0f : 1.0f; /* fp32 quotient */
                ((float *)k_scale)[row] = s;
                for (int d = 0; d < D; ++d) {
                    float v = x[d] / s; /* fp32 quotient */
                    ((uint8_t *)k_cache)[row * D + d] = e4m3_of(v);
                }
            } else {
                for (int blk = 0; blk < D / 32; ++blk) {
                    float amax = 0.0f;
                    for (int d = 32 * blk; d < 32 * blk + 32; ++d)
                        amax = fabsf(x[d]) > amax ? fabsf(x[d]) : amax;
                    int e = 0;
                    if (amax > 0.0f) {
                        int ex;
                        frexp(amax, &ex);
                        e = ex - 1 - 8; /* floor(log2 amax) minus e4m3's largest exponent */
                        e = e < -127 ? -127 : (e > 127 ? 127 : e);
                    }
                    ((uint8_t *)k_scale)[row * (D / 32) + blk] = (uint8_t)(e + 127);
                    for (int d = 32 * blk; d < 32 * blk + 32; ++d)
                        ((uint8_t *)k_cache)[row * D + d] = e4m3_of(ldexp((double)x[d], -e)); /* exact scaling */
                }
            }
        }
    }
    free(x);
    return 0;
}

/* ---- Latent cache append: the new token's row of the main attention cache --
 * Besides the indexer key, each new token leaves one latent row (Dv latent
 * dims, then the rope dims) in the paged cache that sparse attention reads
 * ("Optimizing Inference for Hybrid Attention Architectures: From Operator
 * Fusion to Sequence Sharding", section "Breaking Down the Computational Path
 * of Hybrid Attention", item 2: the main attention cache).  Placement is the
 * indexer append's: row j of request b's new rows goes to position
 * L_b - n_b + j.  dst_dtype 0 copies fp32 rows, 1 rounds to bf16 (nearest
 * even).  dst_dtype 2 writes the fp8 latent row read by sparse attention
 * ("Day0 Inference Optimization for Next-Generation Hybrid-Architecture LLMs
 * Based on CANN", section 3.2: FP8 per token and per 128-element tile):
 * for tile t (latent dims 128t .. 128t + 127) the exponent e is the smallest
 * integer with amax <= 448 * 2^e (e = 0 for a zero tile), clamped to
 * [-126, 127]; byte t of the 16-byte scale block is e + 127 (the other bytes
 * are 0); the codes are the e4m3 codes of x * 2^-e (exact); the rope dims
 * follow as bf16 (nearest even). */
static int tile_exponent(double amax)
{
    if (amax == 0.0)
        return 0;
    int e = ilogb(amax) - 8; /* a start near the answer; the loops fix it exactly */
    while (amax > ldexp(448.0, e))
        ++e;
    while (amax <= ldexp(448.0, e - 1))
        --e;
    return e < -126 ? -126 : (e > 127 ? 127 : e);
}

int dsa_oracle_latent_append(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                             const int32_t *block_table, int bt_stride, int page_size, int Dqk, int Dv,
                             int src_dtype, const void *x_new, int dst_dtype, void *kv_cache)
{
    if (B < 1 || Dqk < 1 || Dv < 1 || Dv > Dqk || page_size < 1 || !q_offsets || !ctx_lens || !block_table ||
        !x_new || !kv_cache)
        return -1;
    if ((src_dtype != 0 && src_dtype != 1) || dst_dtype < 0 || dst_dtype > 2)
        return -1;
    if (dst_dtype == 2 && (Dv % 128 != 0 || Dv / 128 > 16))
        return -1;
    size_t row_bytes = dst_dtype == 2 ? (size_t)Dv + 16 + 2 * (size_t)(Dqk - Dv)
                                      : (size_t)Dqk * (dst_dtype == 0 ? 4 : 2);
    float *x = malloc(sizeof(float) * (size_t)Dqk);
    if (!x)
        return -2;
    for (int b = 0; b < B; ++b) {
        int n = q_offsets[b + 1] - q_offsets[b], L = ctx_lens[b];
        if (n < 0 || n > L) {
            free(x);
            return -1;
        }
        for (int j = 0; j < n; ++j) {
            size_t i = (size_t)q_offsets[b] + j;
            int p = L - n + j;
            int page = block_table[(size_t)b * bt_stride + p / page_size];
            unsigned char *r = (unsigned char *)kv_cache + ((size_t)page * page_size + p % page_size) * row_bytes;
            for (int d = 0; d < Dqk; ++d)
                x[d] = (float)load_elem(x_new, i * Dqk + d, src_dtype); /* exact */
            if (dst_dtype == 0) {
                memcpy(r, x, sizeof(float) * (size_t)Dqk);
            } else if (dst_dtype == 1) {
                for (int d = 0; d < Dqk; ++d) {
                    uint16_t h = dsa_oracle_encode_bf16(x[d]);
                    memcpy(r + 2 * (size_t)d, &h, sizeof h);
                }
            } else {
                memset(r + Dv, 0, 16);
                for (int t = 0; t < Dv / 128; ++t) {
                    double amax = 0.0;
                    for (int d = 128 * t; d < 128 * t + 128; ++d)
                        amax = fabs((double)x[d]) > amax ? fabs((double)x[d]) : amax;
                    int e = tile_exponent(amax);
                    r[Dv + t] = (uint8_t)(e + 127);
                    for (int d = 128 * t; d < 128 * t + 128; ++d)
                        r[d] = e4m3_of(ldexp((double)x[d], -e));
                }
                for (int d = Dv; d < Dqk; ++d) {
                    uint16_t h = dsa_oracle_encode_bf16(x[d]);
                    memcpy(r + Dv + 16 + 2 * (size_t)(d - Dv), &h, sizeof h);
                }
            }
        }
    }
    free(x);
    return 0;
}
