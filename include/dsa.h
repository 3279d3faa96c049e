/*
 * dsa.h -- C ABI of the MI355X (gfx950) DSA sparse-attention step.
 *
 * The step has three parts, after "Optimizing Inference for Hybrid Attention
 * Architectures: From Operator Fusion to Sequence Sharding", section
 * "Breaking Down the Computational Path of Hybrid Attention":
 *   1. the lightning indexer scores every visible cached position against the
 *      query, per indexer head, and weights the heads by importance:
 *          s_t = sum_h w_h * max(q_h . k_t, 0)
 *   2. it keeps the Top-K positions as sparse indices;
 *   3. sparse flash attention reads only those rows of the latent KV cache and
 *      runs softmax attention over them.
 * Parts 1-2 read the paged K cache directly and write only indices ("Day0
 * Inference Support and Performance Optimization for New LLM Architectures",
 * section III, 3.1); part 3 gathers the selected rows from the paged main
 * cache (same page, section III, 3.2).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every array pointer is DEVICE memory owned by the caller; the
 *   library never allocates, frees, copies host<->device or synchronizes.
 *   Descriptor structs themselves are host memory, read during the call only.
 * Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *   Calls only enqueue work on it and return; results are visible once the
 *   stream has reached that point.
 * Workspace: `ws` is caller-owned device memory of at least the size the
 *   matching *_workspace_size call returns, 256-byte aligned.  It must be
 *   zero-filled once before its first use (dsa_workspace_init does that with
 *   a kernel, no memset node); every call leaves its counters and histograms
 *   zero again, so a workspace is reused across calls without re-filling.
 *   Concurrent calls must not share a workspace.
 * Errors: arguments are validated on the host before anything is enqueued;
 *   on a bad argument the call returns a non-zero dsa_status_t and enqueues
 *   nothing.  Device data (page ids, lengths) is trusted: a page id outside
 *   [0, num_pages) or a ctx_len above max_ctx_len is undefined behaviour.
 *   dsa_validate_paged checks that data on the device, on request.
 * Layouts (row-major, contiguous):
 *   paged pools      [num_pages][page_size][dim]        page_size = 64
 *   block_table      [batch][max_pages_per_req] int32   physical page ids
 *   q_offsets        [batch+1] int32; request b owns query rows
 *                    [q_offsets[b], q_offsets[b+1]) (non-decreasing, q_offsets[0] = 0)
 *   ctx_lens         [batch] int32; L_b includes request b's own query tokens,
 *                    so its n_b query rows sit at positions L_b-n_b .. L_b-1
 *                    and row j sees positions 0 .. L_b-n_b+j (causal).
 *   fp8 storage      OCP e4m3 (no infinities) codes; value = code * fp32 scale.
 *   bf16 storage     raw 16-bit patterns.
 * Indices: logical positions within the request (not physical slots),
 *   ascending, padded with -1 when fewer than K positions are visible.
 *   Equal scores at the K-th place: the lower position is kept.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1
#define DSA_PAGE_SIZE 64

typedef enum {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = 1,       /* null pointer, bad size or bad combination */
    DSA_ERR_UNSUPPORTED = 2,       /* valid but not implemented (dims, dtype) */
    DSA_ERR_WORKSPACE_TOO_SMALL = 3,
    DSA_ERR_LAUNCH = 4,            /* the HIP runtime refused a launch */
    DSA_ERR_DEVICE = 5,            /* no usable gfx950 device current */
    DSA_ERR_SCRATCH_LIMIT = 6      /* dsa_fused_decode_static: more scratch needed than
                                      DSA_STATIC_SCRATCH_BYTES */
} dsa_status_t;

/* DSA_MXFP8: e4m3 codes with one E8M0 scale byte (value 2^(E - 127)) per 32
 * consecutive elements of each q (row, head) and each key, the MXFP8
 * grouping of the indexer's q and k ("Optimizing Inference for Hybrid
 * Attention Architectures: From Operator Fusion to Sequence Sharding",
 * section "Layered Quantization: Distinguishing Precision Sensitivity"). */
typedef enum { DSA_F32 = 0, DSA_BF16 = 1, DSA_FP8_E4M3 = 2, DSA_MXFP8 = 3 } dsa_dtype_t;

/* Paging and batch description, shared by both caches (one block table and
 * one page size for the indexer K pool and the latent pool). */
typedef struct {
    int32_t batch;             /* B >= 1 */
    int32_t num_q_tokens;      /* T = q_offsets[B] >= 1 */
    int32_t max_q_per_req;     /* host bound >= every n_b (sizes grids) */
    int32_t max_ctx_len;       /* host bound >= every L_b */
    int32_t max_pages_per_req; /* block-table row stride >= ceil(max_ctx_len / 64) */
    int32_t page_size;         /* must be 64 */
    int32_t num_pages;         /* pages in each pool */
    const int32_t *q_offsets;  /* device [B+1] */
    const int32_t *ctx_lens;   /* device [B] */
    const int32_t *block_table;/* device [B][max_pages_per_req] */
} dsa_paged_t;

/* Lightning indexer.  Supported: head_dim in {64, 128} for F32, BF16 and
 * FP8_E4M3 (F32 also needs n_heads*head_dim <= 4096); MXFP8 with head_dim
 * 128; 1 <= n_heads <= 64; 1 <= topk <= 4096.  Anything else returns
 * DSA_ERR_UNSUPPORTED. */
typedef struct {
    int32_t n_heads;           /* H_I */
    int32_t head_dim;          /* D_I */
    int32_t topk;              /* K */
    int32_t dtype;             /* dsa_dtype_t of q and k_cache */
    const void *q;             /* [T][H_I][D_I] */
    const void *q_scale;       /* FP8_E4M3: fp32 [T][H_I]; MXFP8: E8M0 bytes
                                  [T][H_I][D_I/32], 4-byte aligned; else NULL */
    const float *weights;      /* [T][H_I] head-importance weights */
    const void *k_cache;       /* [num_pages][64][D_I] */
    const void *k_scale;       /* FP8_E4M3: fp32 [num_pages][64]; MXFP8: E8M0
                                  bytes [num_pages][64][D_I/32], 4-byte
                                  aligned; else NULL */
    int32_t flags;             /* 0, or DSA_INDEXER_* flags below */
} dsa_indexer_t;

/* Indexer flag: always take the two-pass route (scoring kernel, then one
 * selection workgroup per row) instead of the single fused kernel.  Results
 * are identical; the fused kernel is used by default when every request has
 * at most 4 query rows and max_ctx_len <= 32768. */
#define DSA_INDEXER_TWO_PASS 1

/* Indexer flags: take the two-pass route and pick its scoring kernel.
 * SCORE_ROWS is the row-tiled MFMA kernel (a workgroup per 4 query rows of a
 * request walks all of the request's positions; BF16/FP8/MXFP8 only, FP32 gives
 * DSA_ERR_UNSUPPORTED); SCORE_POSITIONS is the position-tiled kernel (a
 * workgroup per 256 positions and 4 query rows).  Setting both is
 * DSA_ERR_INVALID_ARG.  Without either the library picks by shape (rows when
 * a request has more than 4 query rows and there are at least 1024 rows).
 * Scores, and so results, are identical on every route. */
#define DSA_INDEXER_SCORE_ROWS 2
#define DSA_INDEXER_SCORE_POSITIONS 4

/* Sparse flash attention over a shared MLA latent cache: the key of a
 * position is its whole row (qk_dim = 576 = 512 latent + 64 rope), the value
 * its first v_dim = 512 entries.  Supported: dtype F32, BF16 or FP8_E4M3,
 * qk_dim 576, v_dim 512, n_heads a multiple of 16 up to 128.
 * FP8_E4M3 is the fp8 latent cache ("Day0 Inference Optimization for
 * Next-Generation Hybrid-Architecture LLMs Based on CANN", section 3.2: one
 * scale per token and 128-element tile): each 656-byte row holds the 512
 * latent dims as e4m3 codes, then a 16-byte block whose byte j is the E8M0
 * exponent E_j of dims 128j .. 128j + 127 (value = code * 2^(E_j - 127);
 * E_j in 1 .. 254; the other 12 bytes are unused), then the 64 rope dims as
 * bf16; q and out are bf16.  code * 2^(E - 127) is exact in bf16. */
typedef struct {
    int32_t n_heads;           /* H_q */
    int32_t qk_dim;            /* 576 */
    int32_t v_dim;             /* 512 */
    int32_t dtype;             /* DSA_F32 or DSA_BF16 (q, kv_cache and out),
                                  or DSA_FP8_E4M3 (fp8 latent rows, bf16 q/out) */
    float scale;               /* softmax scale, e.g. 1/sqrt(576) */
    const void *q;             /* [T][H_q][qk_dim] */
    const void *kv_cache;      /* [num_pages][64][qk_dim] (FP8_E4M3: [num_pages][64]
                                  656-byte rows, 16-byte aligned) */
    void *out;                 /* [T][H_q][v_dim], same dtype */
    float *lse;                /* [T][H_q] natural-log sum-exp, or NULL */
} dsa_sfa_t;

/* Bytes of workspace dsa_indexer_topk needs for these arguments (0 when the
 * arguments are invalid). */
size_t dsa_indexer_topk_workspace_size(const dsa_paged_t *paged, const dsa_indexer_t *idx);

/* Steps 1-2: Top-K positions of every query row.  topk_idx is device
 * [T][topk] int32 (written in full). */
dsa_status_t dsa_indexer_topk(const dsa_paged_t *paged, const dsa_indexer_t *idx,
                              int32_t *topk_idx, void *ws, size_t ws_bytes, void *stream);

/* Steps 1-2 up to the weighted scores, without selection: for every query
 * row i (position pos_i = L_b - n_b + j) and every t <= pos_i,
 * scores[i * score_stride + t] = sum_h w_h * max(q_h . k_t, 0) (fp8: the
 * scaled form), in fp32 ("Optimizing Inference for Hybrid Attention
 * Architectures: From Operator Fusion to Sequence Sharding", section
 * "Breaking Down the Computational Path of Hybrid Attention", item 1).
 * scores is device [T][score_stride] fp32 with score_stride >= max_ctx_len;
 * entries t > pos_i are not written.  The values are bit-identical to the
 * ones dsa_indexer_topk selects from (it is its scoring kernel alone, taken
 * as the flags choose; DSA_INDEXER_TWO_PASS has no effect).  Needs no
 * workspace.  INVALID_ARG for a NULL scores or a short score_stride. */
dsa_status_t dsa_indexer_scores(const dsa_paged_t *paged, const dsa_indexer_t *idx,
                                float *scores, int64_t score_stride, void *stream);

/* Indexer cache append: writes each new token's indexer key into the paged K
 * pool, quantized for a low-precision indexer ("Optimizing Inference for
 * Hybrid Attention Architectures: From Operator Fusion to Sequence
 * Sharding", section "Breaking Down the Computational Path of Hybrid
 * Attention", where the normalised key of a new token goes to the indexer's
 * K cache; section "Layered Quantization: Distinguishing Precision
 * Sensitivity" for the MXFP8 grouping).
 * The n_b new keys of request b (rows q_offsets[b] .. q_offsets[b+1]-1 of
 * k_new) are its query tokens: key j goes to position p = L_b - n_b + j, page
 * block_table[b][p / 64], slot p % 64, where dsa_indexer_topk reads it.
 * Per dst_dtype:
 *   F32: copied.  BF16: rounded to nearest even.
 *   FP8_E4M3: k_scale[page][slot] = amax / 448 in fp32 (1 for a zero key);
 *     codes = e4m3 of the fp32 quotient x / scale.
 *   MXFP8 (head_dim 128): per 32-element block, exponent e = floor(log2
 *     amax) - 8 (0 for a zero block), k_scale byte e + 127; codes = e4m3 of
 *     x * 2^-e.
 *   e4m3 codes round to nearest even, saturate at +-448 and keep the sign
 *   of zero.
 * Other slots are not touched.  A key whose position or page falls outside
 * [0, max_ctx_len) or [0, num_pages) is skipped.  Needs no workspace.  An
 * append and an indexer call that reads the same pages must be ordered by
 * the caller (one stream).  INVALID_ARG for NULL pointers or bad dtypes;
 * UNSUPPORTED for head_dim other than 64 or 128 (MXFP8: 128). */
typedef struct {
    int32_t head_dim;          /* D_I */
    int32_t src_dtype;         /* DSA_F32 or DSA_BF16 */
    int32_t dst_dtype;         /* dsa_dtype_t of the cache */
    const void *k_new;         /* [T][D_I] */
    void *k_cache;             /* [num_pages][64][D_I] */
    void *k_scale;             /* FP8_E4M3: fp32 [num_pages][64]; MXFP8: E8M0
                                  bytes [num_pages][64][D_I/32]; else NULL */
} dsa_cache_append_t;

dsa_status_t dsa_indexer_cache_append(const dsa_paged_t *paged, const dsa_cache_append_t *append,
                                      void *stream);

/* Latent cache append: writes each new token's latent row (qk_dim = 576: the
 * 512 latent dims, then the 64 rope dims) into the paged latent pool that
 * dsa_sparse_attn gathers from ("Optimizing Inference for Hybrid Attention
 * Architectures: From Operator Fusion to Sequence Sharding", section
 * "Breaking Down the Computational Path of Hybrid Attention", item 2: the
 * main attention cache; "Day0 Inference Optimization for Next-Generation
 * Hybrid-Architecture LLMs Based on CANN", section 3.2 for the fp8 rows).
 * Placement is dsa_indexer_cache_append's: row j of request b (rows
 * q_offsets[b] .. q_offsets[b+1]-1 of x_new) goes to position
 * p = L_b - n_b + j, page block_table[b][p / 64], slot p % 64.
 * Per dst_dtype:
 *   F32: copied.  BF16: rounded to nearest even.
 *   FP8_E4M3: the 656-byte fp8 latent row of dsa_sfa_t: for each tile t of
 *     128 latent dims, e_t = the smallest integer with amax <= 448 * 2^e_t
 *     (0 for a zero tile, at least -126); the codes are the e4m3 codes of
 *     x * 2^-e_t (nearest even, exact scaling); byte t of the 16-byte block
 *     after the codes is e_t + 127 and its other 12 bytes are 0; the 64 rope
 *     dims follow in bf16 (nearest even).
 * Other rows are not touched.  A row whose position or page falls outside
 * [0, max_ctx_len) or [0, num_pages) is skipped.  Needs no workspace.  The
 * indexer append and this one touch different pools and may run on two
 * streams at once; either must be ordered before the calls that read it.
 * INVALID_ARG for NULL pointers or bad dtypes; UNSUPPORTED for qk_dim other
 * than 576 or v_dim other than 512. */
typedef struct {
    int32_t qk_dim;            /* 576 */
    int32_t v_dim;             /* 512 */
    int32_t src_dtype;         /* DSA_F32 or DSA_BF16 */
    int32_t dst_dtype;         /* DSA_F32, DSA_BF16 or DSA_FP8_E4M3 (the pool's dtype) */
    const void *x_new;         /* [T][qk_dim] */
    void *kv_cache;            /* [num_pages][64][qk_dim] (FP8_E4M3: [num_pages][64]
                                  656-byte rows, 16-byte aligned) */
} dsa_latent_append_t;

dsa_status_t dsa_latent_cache_append(const dsa_paged_t *paged, const dsa_latent_append_t *append,
                                     void *stream);

size_t dsa_sparse_attn_workspace_size(const dsa_paged_t *paged, const dsa_sfa_t *sfa,
                                      int32_t topk);

/* Step 3: attention of every query row over its topk_idx row (device
 * [T][topk] int32 of logical positions, -1 entries skipped; a row with no
 * valid entry yields a zero output and lse = -inf). */
dsa_status_t dsa_sparse_attn(const dsa_paged_t *paged, const dsa_sfa_t *sfa,
                             const int32_t *topk_idx, int32_t topk,
                             void *ws, size_t ws_bytes, void *stream);

size_t dsa_fused_decode_workspace_size(const dsa_paged_t *paged, const dsa_indexer_t *idx,
                                       const dsa_sfa_t *sfa);

/* Steps 1-3 in one call.  topk_idx may be NULL (indices then live only in
 * the workspace); otherwise it receives the indices as dsa_indexer_topk
 * would.  Results equal dsa_indexer_topk followed by dsa_sparse_attn. */
dsa_status_t dsa_fused_decode(const dsa_paged_t *paged, const dsa_indexer_t *idx,
                              const dsa_sfa_t *sfa, int32_t *topk_idx,
                              void *ws, size_t ws_bytes, void *stream);

/* dsa_fused_decode for callers that cannot allocate device memory: code
 * under HIP graph capture, serving loops that forbid allocation, harnesses
 * that ban hipMalloc.  It takes no workspace: its scratch is one static
 * device array of DSA_STATIC_SCRATCH_BYTES per GPU, which the library holds
 * from its first use on that GPU until the process ends.  The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine) and clears
 * the scratch words that must start at zero with a fill kernel on `stream`
 * before its kernels run.  Every call on one GPU shares that GPU's array, so
 * calls that overlap in time on one GPU race: the caller orders them (one
 * stream, or events).  Results, arguments and errors are dsa_fused_decode's,
 * plus DSA_ERR_SCRATCH_LIMIT (returned before any device work) when
 * dsa_fused_decode_workspace_size of the same arguments exceeds
 * DSA_STATIC_SCRATCH_BYTES. */
#define DSA_STATIC_SCRATCH_BYTES (64u << 20)
dsa_status_t dsa_fused_decode_static(const dsa_paged_t *paged, const dsa_indexer_t *idx,
                                     const dsa_sfa_t *sfa, int32_t *topk_idx, void *stream);

/* Device-side check of the paging data every other call trusts (the block
 * table maps position t of request b to page block_table[b][t / 64], slot
 * t % 64: "Optimizing Inference for Hybrid Attention LLMs: Practices for Fast
 * Adaptation", section 3.2; "Day0 Inference Support and Performance
 * Optimization for New LLM Architectures", section III, 3.2).  One kernel
 * enqueued on `stream` reads q_offsets, ctx_lens and the used entries of
 * block_table (pages 0 .. ceil(ctx_len / 64) - 1 of each request, never past
 * max_pages_per_req) and stores into *error_word (device, 4-byte aligned,
 * overwritten: it needs no clearing) the OR of:
 *   DSA_VALID_Q_OFFSETS  q_offsets[0] != 0, q_offsets[batch] != num_q_tokens,
 *                        or q_offsets decreasing
 *   DSA_VALID_ROWS       a request with more than max_q_per_req rows
 *   DSA_VALID_CTX_LEN    ctx_len below the request's rows or above max_ctx_len
 *   DSA_VALID_PAGE_COUNT ceil(ctx_len / 64) above max_pages_per_req
 *   DSA_VALID_PAGE_ID    a used block-table entry outside [0, num_pages)
 * 0 means the data meets the contract of the other calls.  Reads nothing else
 * (no cache, query or index array), so it is safe on any data.  Needs no
 * workspace.  INVALID_ARG for invalid paged arguments or a NULL or misaligned
 * error_word. */
#define DSA_VALID_Q_OFFSETS 1u
#define DSA_VALID_ROWS 2u
#define DSA_VALID_CTX_LEN 4u
#define DSA_VALID_PAGE_COUNT 8u
#define DSA_VALID_PAGE_ID 16u
dsa_status_t dsa_validate_paged(const dsa_paged_t *paged, uint32_t *error_word, void *stream);

/* Zero-fill a workspace (enqueued on `stream`).  ws_bytes % 4 == 0. */
dsa_status_t dsa_workspace_init(void *ws, size_t ws_bytes, void *stream);

const char *dsa_status_string(dsa_status_t status);
int32_t dsa_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
