/*
 * dsa_oracle.h -- CPU oracle of the DSA sparse-attention step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously correct
 * reference that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It shares
 * no code, header, table or helper with the GPU library, and the GPU library
 * never calls it.
 *
 * What it computes follows the pages:
 *   "Optimizing Inference for Hybrid Attention Architectures: From Operator
 *    Fusion to Sequence Sharding", section "Breaking Down the Computational
 *    Path of Hybrid Attention", phases 1 (Index Screening) and 2 (Sparse
 *    Attention Computation);
 *   "Day0 Inference Support and Performance Optimization for New LLM
 *    Architectures", section III, 3.1 (Integrated Indexer Fusion) and 3.2
 *    (Sparse Attention Kernel).
 * The pages give the steps in prose only; the exact score formula
 *   s_t = sum_h w_h * max(q_h . k_t, 0)
 * the tie rule (equal scores: the lower position wins), the causal visibility
 * rule and the output order (ascending positions, then -1) are the readings
 * this oracle takes from that prose.  Every floating-point step runs in fp64.
 *
 * Storage conventions (identical to the GPU library's, restated here so the
 * oracle stands alone):
 *   dtype 0 = fp32, 1 = bf16 (raw 16-bit patterns), 2 = fp8 e4m3 (OCP "fn"
 *   encoding, raw bytes; real value = code * fp32 scale), 3 = MXFP8 (e4m3
 *   codes; one E8M0 scale byte per 32 consecutive elements of a vector, real
 *   value = code * 2^(E - 127)).
 *   Paged pools are [num_pages][page_size][dim]; block_table is
 *   [B][bt_stride] of physical page ids; request b owns query rows
 *   [q_offsets[b], q_offsets[b+1]) and L_b = ctx_lens[b] cached positions,
 *   which include its own query tokens, so query row j of request b sits at
 *   position L_b - n_b + j and sees positions 0..L_b - n_b + j.
 *
 * Every function returns 0 on success and a negative value on a bad argument.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Decode one stored element to fp64. */
double dsa_oracle_decode_bf16(uint16_t bits);
double dsa_oracle_decode_e4m3(uint8_t code);
double dsa_oracle_decode_e8m0(uint8_t code);

/* Number of positions query row i may see (pos_i + 1), for all rows.
 * vis[T]; T = q_offsets[B]. */
int dsa_oracle_visible(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                       int32_t *vis);

/* Lightning-indexer scores, fp64.  scores is [T][L_out]; entry [i][t] is the
 * score of position t for query row i when t is visible to row i, and NaN
 * otherwise (and for t >= L_out).  L_out must be >= every row's visible count.
 * q is [T][H][D], q_scale [T][H] fp32 (fp8) or [T][H][D/32] E8M0 bytes
 * (MXFP8), w [T][H] fp32, k_cache [num_pages][page_size][D], k_scale
 * [num_pages][page_size] fp32 (fp8) or [num_pages][page_size][D/32] bytes. */
int dsa_oracle_scores(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                      const int32_t *block_table, int bt_stride, int page_size,
                      int H, int D, int dtype,
                      const void *q, const void *q_scale, const float *w,
                      const void *k_cache, const void *k_scale,
                      int L_out, double *scores, int nthreads);

/* Top-K of each row of a score matrix: the first min(K, vis[i]) positions in
 * the order (score descending, position ascending), written in ascending
 * position order and padded with -1.  idx is [T][K]. */
int dsa_oracle_select(int T, int L_out, const double *scores, const int32_t *vis,
                      int K, int32_t *idx, int nthreads);

/* Scores then selection; scores_out may be NULL. */
int dsa_oracle_indexer_topk(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                            const int32_t *block_table, int bt_stride, int page_size,
                            int H, int D, int dtype,
                            const void *q, const void *q_scale, const float *w,
                            const void *k_cache, const void *k_scale,
                            int K, int32_t *idx, int L_out, double *scores_out,
                            int nthreads);

/* Sparse attention over the selected positions.  q is [T][H][Dqk]; kv_cache is
 * [num_pages][page_size][Dqk]; the key of position t is its whole row, the
 * value its first Dv entries.  idx is [T][K] of logical positions (-1 = none).
 * out is [T][H][Dv] fp64, lse [T][H] fp64 (natural log; -inf and a zero
 * output for a row with no selected position).  lse may be NULL. */
int dsa_oracle_sparse_attn(int B, const int32_t *q_offsets,
                           const int32_t *block_table, int bt_stride, int page_size,
                           int H, int Dqk, int Dv, int dtype, double scale,
                           const void *q, const void *kv_cache,
                           const int32_t *idx, int K,
                           double *out, double *lse, int nthreads);

/* Encode one fp32 value: e4m3 (nearest even, saturating at +-448, the sign
 * kept on zero) and bf16 (nearest even). */
uint8_t dsa_oracle_encode_e4m3(float x);
uint16_t dsa_oracle_encode_bf16(float x);

/* Cache append: the n_b new keys of request b (k_new rows q_offsets[b] ..,
 * [T][D] fp32 or bf16, src_dtype 0 or 1) are written to positions
 * L_b - n_b + j of the paged K pool in dst_dtype: fp32 copied; bf16 rounded
 * to nearest even; fp8 with a per-token fp32 scale amax / 448 (1 for a zero
 * key) into k_scale [num_pages][page_size] and codes of the fp32 quotients;
 * MXFP8 with one E8M0 byte per 32-element block (exponent floor(log2 amax)
 * - 8, 0 for a zero block) into k_scale [num_pages][page_size][D/32] and codes
 * of x * 2^-exponent.  Codes round to nearest even and saturate at +-448.
 * Every other slot of the pools is left as it was. */
int dsa_oracle_cache_append(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                            const int32_t *block_table, int bt_stride, int page_size, int D,
                            int src_dtype, const void *k_new, int dst_dtype,
                            void *k_cache, void *k_scale);

/* Latent cache append: the n_b new rows of request b (x_new rows
 * q_offsets[b] .., [T][Dqk] fp32 or bf16, src_dtype 0 or 1) are written to
 * positions L_b - n_b + j of the latent pool in dst_dtype: 0 fp32 rows of Dqk
 * elements, copied; 1 bf16 rows, rounded to nearest even; 2 fp8 latent rows
 * of Dv + 16 + 2 (Dqk - Dv) bytes: Dv e4m3 codes of x * 2^-e_t, where e_t is
 * the smallest integer with amax of 128-element tile t <= 448 * 2^e_t (0 for
 * a zero tile, clamped to [-126, 127]), then a 16-byte block whose byte t is
 * e_t + 127 (the rest 0), then the Dqk - Dv rope dims in bf16.  Every other
 * row of the pool is left as it was. */
int dsa_oracle_latent_append(int B, const int32_t *q_offsets, const int32_t *ctx_lens,
                             const int32_t *block_table, int bt_stride, int page_size, int Dqk, int Dv,
                             int src_dtype, const void *x_new, int dst_dtype, void *kv_cache);

#ifdef __cplusplus
}
#endif
#endif
