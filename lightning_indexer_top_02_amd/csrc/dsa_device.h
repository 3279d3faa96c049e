// dsa_device.h -- device helpers and kernel-launcher declarations shared by
// the HIP sources of the DSA step library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dsa {

constexpr int kPage = 64;          // tokens per cache page
constexpr int kQkDim = 576;        // latent (512) + rope (64)
constexpr int kVDim = 512;
constexpr int kHistBins = 2048;    // bins of the widest radix digit (11 bits)
constexpr int kHistStride = 3 * kHistBins;  // per-row digit histograms in the workspace

// Flag bits of dsa_validate_paged (the same values as the DSA_VALID_* macros
// of the public header).
constexpr uint32_t kValidQOffsets = 1u;   // q_offsets[0] != 0, a decrease, or q_offsets[batch] != T
constexpr uint32_t kValidRows = 2u;       // a request with more than max_q_per_req rows
constexpr uint32_t kValidCtxLen = 4u;     // ctx_len below its rows or above max_ctx_len
constexpr uint32_t kValidPageCount = 8u;  // more pages than max_pages_per_req
constexpr uint32_t kValidPageId = 16u;    // a used block-table entry outside [0, num_pages)

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;

// ---------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Order-preserving 32-bit key of an fp32 score: a larger score gives a larger
// unsigned key; -0 and +0 map to the same key, so equal scores tie exactly.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---------------------------------------------------------------------------
// Reductions over the four 16-lane groups of a wave (lane l, l ^ 16, l ^ 32,
// l ^ 48: one column of an MFMA 16x16 result), with the VALU row permutes of
// gfx950 instead of LDS shuffles.  v_permlane16_swap exchanges rows 1 and 3
// of its first operand with rows 0 and 2 of its second, so swapping a value
// with itself leaves the row pair (2k, 2k+1) in the two outputs, in that
// order on every lane; v_permlane32_swap does the same for the two halves.
// Every lane gets (x0 op x1) op (x2 op x3), with xg the value of group g.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Four such sums at once, each left in one lane group: lane group g returns
// the sum of x[g] over the four groups, formed in group4_sum's pairing and
// order (so bit-identical to it).  The first swaps pair x[0] with x[1] and
// x[2] with x[3], leaving even groups the partial sums of x[0] and x[2] and
// odd groups those of x[1] and x[3]; the half swap then splits each pair.
// Three swaps and three adds where four group4_sum calls take eight of each.
__device__ __forceinline__ float group4_sum_scatter(const float (&x)[4]) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[0]), __float_as_uint(x[1]), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x[2]), __float_as_uint(x[3]), false, false);
  const float s01 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float s23 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s01), __float_as_uint(s23), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

__device__ __forceinline__ float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// ---------------------------------------------------------------------------
// Wave scans through DPP (the VALU's data-parallel-primitive operand
// routing of the GFX9 family) instead of LDS shuffles.  update_dpp(0, x, ...)
// hands each lane the routed value of x, or 0 where the route has no source
// lane or the lane's row is masked off.
//   row_shr:n (0x110 + n)  lane l of a 16-lane row gets lane l - n of that row
//   row_bcast:15 (0x142)   every lane of row r gets lane 15 of row r - 1
//   row_bcast:31 (0x143)   every lane of rows 2 and 3 gets lane 31
// All 64 lanes must be active.
// ---------------------------------------------------------------------------
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ int dpp_route(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, ROW_MASK, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes in lane order: a Hillis-Steele scan
// inside each 16-lane row, then the totals of rows 0 and 2 added to rows 1
// and 3, then the total of rows 0-1 added to rows 2 and 3.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += dpp_route<0x111>(x);
  x += dpp_route<0x112>(x);
  x += dpp_route<0x114>(x);
  x += dpp_route<0x118>(x);
  x += dpp_route<0x142, 0xa>(x);
  x += dpp_route<0x143, 0xc>(x);
  return x;
}

// x of lane l ^ off within each group of four lanes (off = 1 or 2), with a
// quad_perm route: 0xB1 sends lanes (1, 0, 3, 2) to (0, 1, 2, 3), 0x4E sends
// lanes (2, 3, 0, 1).
__device__ __forceinline__ float quad_xor(float x, int off) {
  const int v = __float_as_int(x);
  return __int_as_float(off == 1 ? dpp_route<0xB1>(v) : dpp_route<0x4E>(v));
}

// Value of x on lane `src` (wave-uniform), through a scalar register.
__device__ __forceinline__ int wave_read_lane(int x, int src) { return __builtin_amdgcn_readlane(x, src); }

// ---------------------------------------------------------------------------
// Request lookup: the request that owns query row i (q_offsets is sorted).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int request_of_row(const int32_t* q_offsets, int batch, int i) {
  int lo = 0, hi = batch - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (q_offsets[mid] <= i) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace dsa

// ---------------------------------------------------------------------------
// Launchers (host side).  Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------
struct DsaIndexerLaunch {
  int batch, num_rows, max_q_per_req, max_ctx_len, bt_stride;
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* block_table;
  int n_heads, head_dim, topk, dtype;
  const void* q;
  const void* q_scale;   // fp8: fp32 [T][H]; MXFP8: E8M0 bytes [T][H][D/32]
  const float* weights;
  const void* k_cache;
  const void* k_scale;   // fp8: fp32 [pages][64]; MXFP8: E8M0 bytes [pages][64][D/32]
  int32_t* out_idx;
  // workspace
  uint32_t* counters;  // [batch] arrival counters of the fused kernel, zero between calls
  uint32_t* hist;      // [rows][kHistStride] digit histograms (two-pass), zero between calls; null: scores only
  float* scores;       // [rows][score_stride] scores (two-pass) or score keys (fused)
  int64_t score_stride;
  uint32_t* cand_key;  // [rows][cand_cap] selection candidates (two-pass)
  int32_t* cand_pos;
  int cand_cap;
  uint32_t* keep_bits;  // [rows][dsa_seg_keep_words(score_stride)] kept-position bitmaps (two-pass)
  bool force_two_pass; // skip the fused kernel
  int score_route;     // two-pass scoring: 0 chosen by shape, 1 row-tiled, 2 position-tiled
};

struct DsaSfaLaunch {
  int batch, num_rows;
  const int32_t* q_offsets;
  const int32_t* block_table;
  int bt_stride;
  int n_heads, dtype;
  float scale;
  const void* q;
  const void* kv_cache;
  const int32_t* idx;
  int topk;
  void* out;
  float* lse;
  int nw;  // 16-head tiles per bf16 workgroup (1..4, dividing n_heads / 16)
  // split-KV partials (used when n_split > 1)
  int n_split, rows_per_split;
  uint16_t* part_o;    // [n_split][rows][H][512] fp16 normalised partial outputs
  float* part_lse;     // [n_split][rows][H]
};

// Let `kernel` use `bytes` of dynamic LDS on the current device (above the
// default 64 KB).  The attribute is set once per (device, kernel, size) and
// remembered, so launches do not pay for it every call.
struct DsaAppendLaunch {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* block_table;
  int batch, max_q_per_req, max_ctx_len, bt_stride, num_pages;
  int head_dim, src_dtype, dst_dtype;
  const void* k_new;
  void* k_cache;
  void* k_scale;
};

struct DsaLatentAppendLaunch {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* block_table;
  int batch, max_q_per_req, max_ctx_len, bt_stride, num_pages;
  int src_dtype, dst_dtype;  // src 0 fp32 / 1 bf16; dst 0 fp32, 1 bf16, 2 fp8 latent rows
  const void* x_new;
  void* kv_cache;
};

hipError_t dsa_allow_lds(const void* kernel, size_t bytes);
hipError_t dsa_launch_cache_append(const DsaAppendLaunch& a, hipStream_t s);
hipError_t dsa_launch_latent_append(const DsaLatentAppendLaunch& a, hipStream_t s);

hipError_t dsa_launch_indexer_topk(const DsaIndexerLaunch& a, hipStream_t s);
hipError_t dsa_launch_indexer_two_pass(const DsaIndexerLaunch& a, hipStream_t s);
// Scoring kernel of the two-pass route alone (a.hist may be null: no histograms).
hipError_t dsa_launch_indexer_scores(const DsaIndexerLaunch& a, hipStream_t s);
hipError_t dsa_launch_indexer_prefill_scores(const DsaIndexerLaunch& a, hipStream_t s);
hipError_t dsa_launch_topk_segments(const DsaIndexerLaunch& a, hipStream_t s);
int dsa_seg_max_segments();
int dsa_seg_length();  // positions per selection segment
int dsa_seg_cand_cap(int max_ctx_len);
int64_t dsa_seg_keep_words(int64_t score_stride);  // kept-position bitmap words per row
bool dsa_indexer_rows_route(const DsaIndexerLaunch& a);
hipError_t dsa_launch_sparse_attn(const DsaSfaLaunch& a, hipStream_t s);
hipError_t dsa_launch_validate(const int32_t* q_offsets, const int32_t* ctx_lens, const int32_t* block_table,
                               int batch, int num_q_tokens, int max_q_per_req, int max_ctx_len,
                               int max_pages_per_req, int num_pages, uint32_t* error_word, hipStream_t s);
