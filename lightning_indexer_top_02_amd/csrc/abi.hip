// abi.hip -- the C ABI of include/dsa.h: host-side validation, workspace
// sizing and dispatch to the kernel launchers.  Validation runs before any
// HIP runtime call, so a rejected call touches no device.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "../../include/dsa.h"
#include "dsa_device.h"

namespace {

constexpr int kMaxTopk = 4096;
constexpr int kMaxIdxHeads = 64;
constexpr int kSfaMaxHeads = 128;
constexpr int kNominalCUs = 256;   // MI355X; fixes split choices independently of the device
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

bool valid_paged(const dsa_paged_t* p) {
  if (!p) return false;
  if (p->batch < 1 || p->num_q_tokens < 1 || p->max_q_per_req < 1 || p->max_ctx_len < 1) return false;
  if (p->page_size != DSA_PAGE_SIZE || p->num_pages < 1) return false;
  if (p->max_q_per_req > p->num_q_tokens || p->max_q_per_req > p->max_ctx_len) return false;
  if (p->num_q_tokens < p->batch) return false;
  if ((int64_t)p->max_pages_per_req * DSA_PAGE_SIZE < p->max_ctx_len) return false;
  if (!p->q_offsets || !p->ctx_lens || !p->block_table) return false;
  return true;
}

dsa_status_t check_indexer(const dsa_paged_t* pg, const dsa_indexer_t* x) {
  if (!valid_paged(pg) || !x) return DSA_ERR_INVALID_ARG;
  if (!x->q || !x->weights || !x->k_cache) return DSA_ERR_INVALID_ARG;
  if (x->n_heads < 1 || x->head_dim < 1 || x->topk < 1) return DSA_ERR_INVALID_ARG;
  if (x->dtype != DSA_F32 && x->dtype != DSA_BF16 && x->dtype != DSA_FP8_E4M3 && x->dtype != DSA_MXFP8)
    return DSA_ERR_INVALID_ARG;
  if ((x->dtype == DSA_FP8_E4M3 || x->dtype == DSA_MXFP8) && (!x->q_scale || !x->k_scale))
    return DSA_ERR_INVALID_ARG;
  constexpr int32_t kRouteFlags = DSA_INDEXER_SCORE_ROWS | DSA_INDEXER_SCORE_POSITIONS;
  if (x->flags & ~(DSA_INDEXER_TWO_PASS | kRouteFlags)) return DSA_ERR_INVALID_ARG;
  if ((x->flags & kRouteFlags) == kRouteFlags) return DSA_ERR_INVALID_ARG;
  if (x->n_heads > kMaxIdxHeads || x->topk > kMaxTopk) return DSA_ERR_UNSUPPORTED;
  if (x->head_dim != 64 && x->head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (x->dtype == DSA_MXFP8) {
    // the kernels read a (row, head)'s or a key's four scale bytes as one word
    if ((reinterpret_cast<uintptr_t>(x->q_scale) | reinterpret_cast<uintptr_t>(x->k_scale)) & 3)
      return DSA_ERR_INVALID_ARG;
    if (x->head_dim != 128) return DSA_ERR_UNSUPPORTED;  // one 16x16x128 step
  }
  if (x->dtype == DSA_F32 && x->n_heads * x->head_dim > 4096) return DSA_ERR_UNSUPPORTED;
  if ((int64_t)pg->max_ctx_len > (int64_t)dsa_seg_max_segments() * dsa_seg_length()) return DSA_ERR_UNSUPPORTED;
  if (x->dtype == DSA_F32 && (x->flags & DSA_INDEXER_SCORE_ROWS)) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

dsa_status_t check_sfa(const dsa_paged_t* pg, const dsa_sfa_t* s, int32_t topk) {
  if (!valid_paged(pg) || !s) return DSA_ERR_INVALID_ARG;
  if (!s->q || !s->kv_cache || !s->out) return DSA_ERR_INVALID_ARG;
  if (topk < 1 || s->n_heads < 1 || s->qk_dim < 1 || s->v_dim < 1 || s->v_dim > s->qk_dim)
    return DSA_ERR_INVALID_ARG;
  if (s->dtype != DSA_F32 && s->dtype != DSA_BF16 && s->dtype != DSA_FP8_E4M3) return DSA_ERR_INVALID_ARG;
  if (!std::isfinite(s->scale)) return DSA_ERR_INVALID_ARG;
  if (s->qk_dim != dsa::kQkDim || s->v_dim != dsa::kVDim) return DSA_ERR_UNSUPPORTED;
  if (s->n_heads % 16 != 0 || s->n_heads > kSfaMaxHeads || topk > kMaxTopk) return DSA_ERR_UNSUPPORTED;
  return DSA_OK;
}

// --- workspace plans ---------------------------------------------------------
// Indexer workspace: arrival counters [batch] u32 | digit histograms
// [rows][kHistStride] u32 | scores or score keys [rows][round_up(L_max, 256)].
// The first two regions are zero between calls.
struct IndexerPlan {
  int64_t score_stride;
  int cand_cap;
  size_t ctrl_off, hist_off, scores_off, cand_key_off, cand_pos_off, keep_off, total;
};

IndexerPlan plan_indexer(const dsa_paged_t* pg) {
  IndexerPlan p;
  const size_t T = (size_t)pg->num_q_tokens;
  p.score_stride = round_up(pg->max_ctx_len, 256);
  p.ctrl_off = 0;
  p.hist_off = align_up(4 * (size_t)pg->batch);
  p.scores_off = p.hist_off + align_up(T * dsa::kHistStride * 4);
  p.cand_cap = dsa_seg_cand_cap(pg->max_ctx_len);
  p.cand_key_off = p.scores_off + align_up(T * p.score_stride * 4);
  p.cand_pos_off = p.cand_key_off + align_up(T * (size_t)p.cand_cap * 4);
  p.keep_off = p.cand_pos_off + align_up(T * (size_t)p.cand_cap * 4);
  p.total = p.keep_off + align_up(T * (size_t)dsa_seg_keep_words(p.score_stride) * 4);
  return p;
}

// 16-head tiles per SFA workgroup (waves = 2 per tile): up to 4, dividing the
// head count.  A workgroup of 4 tiles shares each gathered row among 64
// heads, which decides throughput once the batch fills the chip; smaller
// batches are latency-bound, and narrower workgroups (more of them on a
// compute unit) finish sooner although each row is gathered by more of
// them.  By the batch's tiles (rows x 16-head groups), measured at 32K
// decode with 128 heads: at most 8 (one row), 1 tile (16.5 us against 22
// with 4); 16 or 32 (2 or 4 rows), 2 tiles (18.9 and 22.5 us against 22.0
// and 27.7 with 4); 64 and more (8 rows), 4 tiles (26.3 us against 27.9).
int sfa_waves(int n_heads, int64_t num_rows) {
  const int hq = n_heads / 16;
  const int64_t tiles = num_rows * hq;
  const int cap = tiles <= 8 ? 1 : (tiles <= 32 ? 2 : 4);
  for (int nw = cap; nw > 1; --nw)
    if (hq % nw == 0) return nw;
  return 1;
}

struct SfaPlan {
  int n_split, rows_per_split, nw;
  size_t part_o_off, part_lse_off, total;
};

SfaPlan plan_sfa(const dsa_paged_t* pg, const dsa_sfa_t* s, int topk) {
  SfaPlan p{1, topk, 1, 0, 0, 0};
  if (s->dtype == DSA_BF16 || s->dtype == DSA_FP8_E4M3) {  // the fp8 latent route shares the bf16 kernel
    p.nw = sfa_waves(s->n_heads, pg->num_q_tokens);
    const int64_t blocks = (int64_t)pg->num_q_tokens * (s->n_heads / (16 * p.nw));
    // about one workgroup per compute unit: a bf16 SFA workgroup of four
    // tiles holds ~230 VGPRs per lane, so a compute unit runs one at a time
    // and a larger grid only queues a second round (64 decode rows at 32K:
    // 107.6 us with two rounds, 94.2 us with one)
    // (one-tile workgroups, ~79 KB of LDS and 2 waves, fit two to a compute unit)
    const int64_t target = p.nw == 1 ? 2 * kNominalCUs : kNominalCUs;
    int64_t splits = (target + blocks - 1) / blocks;
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, (topk + 63) / 64));
    p.rows_per_split = (int)round_up((topk + splits - 1) / splits, 32);
    p.n_split = (topk + p.rows_per_split - 1) / p.rows_per_split;
  } else {  // fp32: 16 heads per workgroup, splits of whole 16-row chunks, about one workgroup per compute unit
    const int64_t blocks = (int64_t)pg->num_q_tokens * (s->n_heads / 16);
    int64_t splits = (kNominalCUs + blocks - 1) / blocks;
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, (topk + 15) / 16));
    p.rows_per_split = (int)round_up((topk + splits - 1) / splits, 16);
    p.n_split = (topk + p.rows_per_split - 1) / p.rows_per_split;
  }
  if (p.n_split > 1) {
    const size_t th = (size_t)pg->num_q_tokens * s->n_heads;
    p.part_o_off = 0;
    p.part_lse_off = align_up((size_t)p.n_split * th * dsa::kVDim * 2);  // fp16 partial outputs
    p.total = p.part_lse_off + align_up((size_t)p.n_split * th * 4);
  }
  return p;
}

// --- device check --------------------------------------------------------------
dsa_status_t check_device() {
  static int cached[64];  // 0 unknown, 1 ok, 2 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DSA_ERR_DEVICE;
  if (dev < 64 && cached[dev]) return cached[dev] == 1 ? DSA_OK : DSA_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSA_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cached[dev] = ok ? 1 : 2;
  return ok ? DSA_OK : DSA_ERR_DEVICE;
}

DsaIndexerLaunch indexer_args(const dsa_paged_t* pg, const dsa_indexer_t* x, int32_t* out,
                              unsigned char* ws, const IndexerPlan& plan) {
  DsaIndexerLaunch a;
  a.batch = pg->batch;
  a.num_rows = pg->num_q_tokens;
  a.max_q_per_req = pg->max_q_per_req;
  a.max_ctx_len = pg->max_ctx_len;
  a.bt_stride = pg->max_pages_per_req;
  a.q_offsets = pg->q_offsets;
  a.ctx_lens = pg->ctx_lens;
  a.block_table = pg->block_table;
  a.n_heads = x->n_heads;
  a.head_dim = x->head_dim;
  a.topk = x->topk;
  a.dtype = x->dtype;
  a.q = x->q;
  a.q_scale = x->q_scale;
  a.weights = x->weights;
  a.k_cache = x->k_cache;
  a.k_scale = x->k_scale;
  a.out_idx = out;
  a.counters = reinterpret_cast<uint32_t*>(ws + plan.ctrl_off);
  a.hist = reinterpret_cast<uint32_t*>(ws + plan.hist_off);
  a.scores = reinterpret_cast<float*>(ws + plan.scores_off);
  a.score_stride = plan.score_stride;
  a.cand_key = reinterpret_cast<uint32_t*>(ws + plan.cand_key_off);
  a.cand_pos = reinterpret_cast<int32_t*>(ws + plan.cand_pos_off);
  a.keep_bits = reinterpret_cast<uint32_t*>(ws + plan.keep_off);
  a.cand_cap = plan.cand_cap;
  a.force_two_pass = (x->flags & (DSA_INDEXER_TWO_PASS | DSA_INDEXER_SCORE_ROWS | DSA_INDEXER_SCORE_POSITIONS)) != 0;
  a.score_route = (x->flags & DSA_INDEXER_SCORE_ROWS) ? 1 : (x->flags & DSA_INDEXER_SCORE_POSITIONS) ? 2 : 0;
  return a;
}

DsaSfaLaunch sfa_args(const dsa_paged_t* pg, const dsa_sfa_t* s, const int32_t* idx, int topk,
                      unsigned char* ws, const SfaPlan& plan) {
  DsaSfaLaunch a;
  a.batch = pg->batch;
  a.num_rows = pg->num_q_tokens;
  a.q_offsets = pg->q_offsets;
  a.block_table = pg->block_table;
  a.bt_stride = pg->max_pages_per_req;
  a.n_heads = s->n_heads;
  a.dtype = s->dtype;
  a.scale = s->scale;
  a.q = s->q;
  a.kv_cache = s->kv_cache;
  a.idx = idx;
  a.topk = topk;
  a.out = s->out;
  a.lse = s->lse;
  a.n_split = plan.n_split;
  a.nw = plan.nw;
  a.rows_per_split = plan.rows_per_split;
  a.part_o = plan.n_split > 1 ? reinterpret_cast<uint16_t*>(ws + plan.part_o_off) : nullptr;
  a.part_lse = plan.n_split > 1 ? reinterpret_cast<float*>(ws + plan.part_lse_off) : nullptr;
  return a;
}

bool ws_ok(const void* ws, size_t have, size_t need) {
  if (need == 0) return true;
  return ws && have >= need && (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0;
}

__global__ void zero_words(uint32_t* x, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    x[i] = 0u;
}

}  // namespace

namespace {

// Workspace of the fused call: the indexer's, then the indices (when the
// caller passes no topk_idx), then the sparse attention's.
struct FusedPlan {
  IndexerPlan ip;
  SfaPlan sp;
  size_t idx_off, sfa_off, total;
};

FusedPlan plan_fused(const dsa_paged_t* pg, const dsa_indexer_t* x, const dsa_sfa_t* s) {
  FusedPlan f;
  f.ip = plan_indexer(pg);
  f.sp = plan_sfa(pg, s, x->topk);
  f.idx_off = align_up(f.ip.total);
  f.sfa_off = f.idx_off + align_up((size_t)pg->num_q_tokens * x->topk * 4);
  f.total = f.sfa_off + f.sp.total;
  return f;
}

dsa_status_t launch_fused_decode(const dsa_paged_t* pg, const dsa_indexer_t* x, const dsa_sfa_t* s,
                                 int32_t* topk_idx, unsigned char* w, const FusedPlan& fp, hipStream_t hs) {
  int32_t* idx = topk_idx ? topk_idx : reinterpret_cast<int32_t*>(w + fp.idx_off);
  if (dsa_launch_indexer_topk(indexer_args(pg, x, idx, w, fp.ip), hs) != hipSuccess) return DSA_ERR_LAUNCH;
  if (dsa_launch_sparse_attn(sfa_args(pg, s, idx, x->topk, w + fp.sfa_off, fp.sp), hs) != hipSuccess)
    return DSA_ERR_LAUNCH;
  return DSA_OK;
}

// Scratch of dsa_fused_decode_static: one array per device, held until the
// process ends.  Host code never uses the array's name as an address (it is a
// host-side stand-in); the device address comes from hipGetSymbolAddress,
// once per device, with that device current.
constexpr size_t kStaticScratchBytes = (size_t)DSA_STATIC_SCRATCH_BYTES;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[64];

}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

dsa_status_t static_scratch(unsigned char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DSA_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSA_ERR_DEVICE;
    g_scratch_ptr[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

hipError_t dsa_allow_lds(const void* kernel, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  // (device, kernel) -> bytes allowed, in a fixed table: a launch path never
  // allocates, not even host memory
  struct Allowed {
    int dev;
    const void* kernel;
    size_t bytes;
  };
  static std::mutex mu;
  static Allowed done[256];
  static int n_done = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  int at = -1;
  for (int k = 0; k < n_done; ++k)
    if (done[k].dev == dev && done[k].kernel == kernel) {
      if (done[k].bytes >= bytes) return hipSuccess;
      at = k;
    }
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  if (at < 0 && n_done < 256) at = n_done++;
  if (at >= 0) done[at] = Allowed{dev, kernel, bytes};
  return hipSuccess;
}

extern "C" {

dsa_status_t dsa_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || ws_bytes % 4 != 0 || (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0) return DSA_ERR_INVALID_ARG;
  if (ws_bytes == 0) return DSA_OK;
  dsa_status_t st = check_device();
  if (st != DSA_OK) return st;
  const size_t n = ws_bytes / 4;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 2048);
  hipLaunchKernelGGL(zero_words, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint32_t*>(ws), n);
  return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

dsa_status_t dsa_validate_paged(const dsa_paged_t* pg, uint32_t* error_word, void* stream) {
  if (!valid_paged(pg) || !error_word || (reinterpret_cast<uintptr_t>(error_word) & 3)) return DSA_ERR_INVALID_ARG;
  dsa_status_t st = check_device();
  if (st != DSA_OK) return st;
  return dsa_launch_validate(pg->q_offsets, pg->ctx_lens, pg->block_table, pg->batch, pg->num_q_tokens,
                             pg->max_q_per_req, pg->max_ctx_len, pg->max_pages_per_req, pg->num_pages,
                             error_word, static_cast<hipStream_t>(stream)) == hipSuccess
             ? DSA_OK
             : DSA_ERR_LAUNCH;
}

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small or misaligned";
    case DSA_ERR_LAUNCH: return "kernel launch failed";
    case DSA_ERR_DEVICE: return "no gfx950 device is current";
    case DSA_ERR_SCRATCH_LIMIT: return "needs more scratch than the library's static array holds";
  }
  return "unknown status";
}

size_t dsa_indexer_topk_workspace_size(const dsa_paged_t* pg, const dsa_indexer_t* x) {
  if (check_indexer(pg, x) != DSA_OK) return 0;
  return plan_indexer(pg).total;
}

dsa_status_t dsa_indexer_topk(const dsa_paged_t* pg, const dsa_indexer_t* x, int32_t* topk_idx,
                              void* ws, size_t ws_bytes, void* stream) {
  dsa_status_t st = check_indexer(pg, x);
  if (st != DSA_OK) return st;
  if (!topk_idx) return DSA_ERR_INVALID_ARG;
  const IndexerPlan plan = plan_indexer(pg);
  if (!ws_ok(ws, ws_bytes, plan.total)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device()) != DSA_OK) return st;
  DsaIndexerLaunch a = indexer_args(pg, x, topk_idx, static_cast<unsigned char*>(ws), plan);
  return dsa_launch_indexer_topk(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

dsa_status_t dsa_indexer_scores(const dsa_paged_t* pg, const dsa_indexer_t* x, float* scores,
                                int64_t score_stride, void* stream) {
  dsa_status_t st = check_indexer(pg, x);
  if (st != DSA_OK) return st;
  if (!scores || score_stride < pg->max_ctx_len) return DSA_ERR_INVALID_ARG;
  if ((st = check_device()) != DSA_OK) return st;
  DsaIndexerLaunch a = indexer_args(pg, x, nullptr, nullptr, IndexerPlan{});
  a.counters = nullptr;
  a.hist = nullptr;
  a.scores = scores;
  a.score_stride = score_stride;
  return dsa_launch_indexer_scores(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

dsa_status_t dsa_indexer_cache_append(const dsa_paged_t* pg, const dsa_cache_append_t* x, void* stream) {
  if (!valid_paged(pg) || !x || !x->k_new || !x->k_cache) return DSA_ERR_INVALID_ARG;
  if (x->src_dtype != DSA_F32 && x->src_dtype != DSA_BF16) return DSA_ERR_INVALID_ARG;
  if (x->dst_dtype != DSA_F32 && x->dst_dtype != DSA_BF16 && x->dst_dtype != DSA_FP8_E4M3 &&
      x->dst_dtype != DSA_MXFP8)
    return DSA_ERR_INVALID_ARG;
  if ((x->dst_dtype == DSA_FP8_E4M3 || x->dst_dtype == DSA_MXFP8) && !x->k_scale) return DSA_ERR_INVALID_ARG;
  if (x->head_dim != 64 && x->head_dim != 128) return DSA_ERR_UNSUPPORTED;
  if (x->dst_dtype == DSA_MXFP8 && x->head_dim != 128) return DSA_ERR_UNSUPPORTED;
  dsa_status_t st = check_device();
  if (st != DSA_OK) return st;
  DsaAppendLaunch a;
  a.q_offsets = pg->q_offsets;
  a.ctx_lens = pg->ctx_lens;
  a.block_table = pg->block_table;
  a.batch = pg->batch;
  a.max_q_per_req = pg->max_q_per_req;
  a.max_ctx_len = pg->max_ctx_len;
  a.bt_stride = pg->max_pages_per_req;
  a.num_pages = pg->num_pages;
  a.head_dim = x->head_dim;
  a.src_dtype = x->src_dtype;
  a.dst_dtype = x->dst_dtype;
  a.k_new = x->k_new;
  a.k_cache = x->k_cache;
  a.k_scale = x->k_scale;
  return dsa_launch_cache_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

dsa_status_t dsa_latent_cache_append(const dsa_paged_t* pg, const dsa_latent_append_t* x, void* stream) {
  if (!valid_paged(pg) || !x || !x->x_new || !x->kv_cache) return DSA_ERR_INVALID_ARG;
  if (x->src_dtype != DSA_F32 && x->src_dtype != DSA_BF16) return DSA_ERR_INVALID_ARG;
  if (x->dst_dtype != DSA_F32 && x->dst_dtype != DSA_BF16 && x->dst_dtype != DSA_FP8_E4M3)
    return DSA_ERR_INVALID_ARG;
  if (x->qk_dim != dsa::kQkDim || x->v_dim != dsa::kVDim) return DSA_ERR_UNSUPPORTED;
  if (x->dst_dtype == DSA_FP8_E4M3 && (reinterpret_cast<uintptr_t>(x->kv_cache) & 15)) return DSA_ERR_INVALID_ARG;
  dsa_status_t st = check_device();
  if (st != DSA_OK) return st;
  DsaLatentAppendLaunch a;
  a.q_offsets = pg->q_offsets;
  a.ctx_lens = pg->ctx_lens;
  a.block_table = pg->block_table;
  a.batch = pg->batch;
  a.max_q_per_req = pg->max_q_per_req;
  a.max_ctx_len = pg->max_ctx_len;
  a.bt_stride = pg->max_pages_per_req;
  a.num_pages = pg->num_pages;
  a.src_dtype = x->src_dtype;
  a.dst_dtype = x->dst_dtype == DSA_FP8_E4M3 ? 2 : x->dst_dtype;
  a.x_new = x->x_new;
  a.kv_cache = x->kv_cache;
  return dsa_launch_latent_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

size_t dsa_sparse_attn_workspace_size(const dsa_paged_t* pg, const dsa_sfa_t* s, int32_t topk) {
  if (check_sfa(pg, s, topk) != DSA_OK) return 0;
  return plan_sfa(pg, s, topk).total;
}

dsa_status_t dsa_sparse_attn(const dsa_paged_t* pg, const dsa_sfa_t* s, const int32_t* topk_idx,
                             int32_t topk, void* ws, size_t ws_bytes, void* stream) {
  dsa_status_t st = check_sfa(pg, s, topk);
  if (st != DSA_OK) return st;
  if (!topk_idx) return DSA_ERR_INVALID_ARG;
  const SfaPlan plan = plan_sfa(pg, s, topk);
  if (!ws_ok(ws, ws_bytes, plan.total)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device()) != DSA_OK) return st;
  DsaSfaLaunch a = sfa_args(pg, s, topk_idx, topk, static_cast<unsigned char*>(ws), plan);
  return dsa_launch_sparse_attn(a, static_cast<hipStream_t>(stream)) == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

size_t dsa_fused_decode_workspace_size(const dsa_paged_t* pg, const dsa_indexer_t* x, const dsa_sfa_t* s) {
  if (check_indexer(pg, x) != DSA_OK || !x || check_sfa(pg, s, x->topk) != DSA_OK) return 0;
  return plan_fused(pg, x, s).total;
}

dsa_status_t dsa_fused_decode(const dsa_paged_t* pg, const dsa_indexer_t* x, const dsa_sfa_t* s,
                              int32_t* topk_idx, void* ws, size_t ws_bytes, void* stream) {
  dsa_status_t st = check_indexer(pg, x);
  if (st != DSA_OK) return st;
  if ((st = check_sfa(pg, s, x->topk)) != DSA_OK) return st;
  const FusedPlan fp = plan_fused(pg, x, s);
  if (!ws_ok(ws, ws_bytes, fp.total)) return DSA_ERR_WORKSPACE_TOO_SMALL;
  if ((st = check_device()) != DSA_OK) return st;
  return launch_fused_decode(pg, x, s, topk_idx, static_cast<unsigned char*>(ws), fp, static_cast<hipStream_t>(stream));
}

dsa_status_t dsa_fused_decode_static(const dsa_paged_t* pg, const dsa_indexer_t* x, const dsa_sfa_t* s,
                                     int32_t* topk_idx, void* stream) {
  dsa_status_t st = check_indexer(pg, x);
  if (st != DSA_OK) return st;
  if ((st = check_sfa(pg, s, x->topk)) != DSA_OK) return st;
  const FusedPlan fp = plan_fused(pg, x, s);
  if (fp.total > kStaticScratchBytes) return DSA_ERR_SCRATCH_LIMIT;
  if ((st = check_device()) != DSA_OK) return st;
  unsigned char* w = nullptr;
  if ((st = static_scratch(&w)) != DSA_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // The array keeps the previous call's contents, and a call of another
  // shape may have left scores or indices where this call's arrival
  // counters and histograms lie: clear those words (a fill kernel, so the
  // call can be captured in a graph), the rest is written before it is read.
  const size_t ctrl_words = fp.ip.scores_off / 4;
  hipLaunchKernelGGL(zero_words, dim3((unsigned)std::min<size_t>((ctrl_words + 255) / 256, 2048)), dim3(256), 0, hs,
                     reinterpret_cast<uint32_t*>(w), ctrl_words);
  if (hipGetLastError() != hipSuccess) return DSA_ERR_LAUNCH;
  return launch_fused_decode(pg, x, s, topk_idx, w, fp, hs);
}

}  // extern "C"
