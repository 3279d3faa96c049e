// indexer.hip -- lightning indexer, throughput path (gfx950): scores through
// HBM, then one selection workgroup per query row.
//
// Used when rows are too long (or too many per request) for the single fused
// kernel (indexer_fused.hip).  Requests with many query rows (chunked prefill)
// are scored by the row-tiled MFMA kernel of indexer_prefill.hip instead of
// li_score; both write the same scores and histograms.  The scoring follows "Optimizing Inference for
// Hybrid Attention Architectures: From Operator Fusion to Sequence Sharding",
// section "Breaking Down the Computational Path of Hybrid Attention", item 1,
// reading keys straight from the paged K cache ("Day0 Inference Support and
// Performance Optimization for New LLM Architectures", section III, 3.1).
//
// li_score: one workgroup = 4 waves, stepping 4 cache pages (256 positions)
// at a time through its share of all requests' chunks, for up to 4 query rows
// of the request at hand (the rows share one read of the keys).
// It writes fp32 scores and a per-row histogram of the top 11 key bits (LDS,
// then one global atomic per non-empty bin): the first radix level.
//
// Selection runs over segments of each row (topk_seg.hip); li_topk takes the
// rows whose boundary bin holds too many keys for that (heavy ties).
// li_topk: one 1024-thread workgroup per query row.  It finds the bin holding
// the K-th largest key, gathers that bin's keys into LDS, resolves the exact
// K-th key with two more radix levels, then makes one ordered pass keeping
// every larger key and the lowest-position keys equal to the K-th (the tie
// rule), writing positions in ascending order.  It zeroes its histogram row
// on the way out, so the workspace stays ready for the next call.
#include <algorithm>

#include "dsa_device.h"
#include "indexer_common.h"
#include "radix_select.h"

namespace dsa {

struct LiParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* bt;
  int batch, bt_stride;
  int H, Hpad;
  int rcap;  // query rows the LDS layout holds (min(4, max rows per request))
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k;
  const float* k_scale;
  float* scores;
  int64_t score_stride;
  uint32_t* hist;  // [rows][kHistStride]; level-1 digit histogram at offset 0 (null: scores only)
};

constexpr int kRowsPerBlock = 4;
constexpr int kScoreThreads = 256;  // 4 waves, one page each
constexpr int kChunk = 256;         // positions per workgroup and step
// Workgroups the scoring grid aims for: one resident round (two 4-wave
// workgroups per compute unit at up to 256 VGPRs), so each workgroup pays its
// start-up (chunk search, query staging, histogram flush) once over a long
// range (speculative verify, 16 x 256K: 300 us with 2048, 270 us with 512).
constexpr int kScoreTargetWGs = 512;

// Chunks of 256 positions row group y (rows 4y .. 4y + 3) of request b
// covers: every position its last row sees, 0 when the request has no such
// rows.
__device__ __forceinline__ int chunks_of(const LiParams& p, int b, int r0) {
  const int nb = p.q_offsets[b + 1] - p.q_offsets[b];
  if (r0 >= nb) return 0;
  const int pos_max = p.ctx_lens[b] - nb + r0 + min(kRowsPerBlock, nb - r0) - 1;
  return pos_max / kChunk + 1;
}

// The chunks of all requests (for one row group) form one list, split evenly
// over the workgroups of the grid's x dimension, so requests of different
// lengths cost their share and no workgroup waits on a long one.  A
// workgroup walks its range in order: it stages the request's query rows
// (and starts its histogram) when it enters a request, flushes the histogram
// when it leaves, and each wave loads its page of the next chunk while it
// scores the current one.
template <int DT, int D>
__global__ __launch_bounds__(kScoreThreads) void li_score(LiParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ __align__(16) int wsum[kScoreThreads / 64];
  __shared__ int s_b0, s_base0;
  using Gm = IdxGeom<DT, D>;
  unsigned char* qs = smem;
  float* wsm = reinterpret_cast<float*>(smem + (size_t)p.rcap * p.Hpad * Gm::QSTRIDE);
  uint32_t* hl = reinterpret_cast<uint32_t*>(wsm + p.rcap * p.Hpad);
  const int tid = threadIdx.x, wave = tid >> 6;
  const int r0 = blockIdx.y * kRowsPerBlock;

  // total chunks and the request holding this workgroup's first one
  const int per = (p.batch + kScoreThreads - 1) / kScoreThreads;
  const int blo = min(p.batch, tid * per), bhi = min(p.batch, blo + per);
  int local = 0;
  for (int b = blo; b < bhi; ++b) local += chunks_of(p, b, r0);
  int total;
  const int excl = block_excl_scan<kScoreThreads>(local, total, wsum);
  const int f0 = (int)((int64_t)blockIdx.x * total / gridDim.x);
  const int f1 = (int)((int64_t)(blockIdx.x + 1) * total / gridDim.x);
  if (f0 >= f1) return;
  if (excl <= f0 && f0 < excl + local) {
    int b = blo, acc = excl;
    while (acc + chunks_of(p, b, r0) <= f0) acc += chunks_of(p, b++, r0);
    s_b0 = b;
    s_base0 = acc;
  }
  __syncthreads();

  // the request being scored
  int b = s_b0, base = s_base0, q0 = 0, nb = 0, nrows = 0, first_pos = 0, pos_max = -1, nchunks = 0;
  auto enter = [&](int nbq) {
    b = nbq;
    q0 = p.q_offsets[b];
    nb = p.q_offsets[b + 1] - q0;
    nrows = min(kRowsPerBlock, nb - r0);
    first_pos = p.ctx_lens[b] - nb;
    pos_max = first_pos + r0 + nrows - 1;
    nchunks = pos_max / kChunk + 1;
    stage_queries<DT, D, kScoreThreads>(qs, wsm, p.q, p.q_scale, p.w, q0 + r0, nrows, p.H, p.Hpad);
    for (int c = tid; c < nrows * kHistBins; c += kScoreThreads) hl[c] = 0u;
    __syncthreads();
  };
  auto leave = [&]() {
    __syncthreads();
    if (!p.hist) return;
    for (int c = tid; c < nrows * kHistBins; c += kScoreThreads) {
      const uint32_t v = hl[c];
      if (v) {
        const int r = c / kHistBins, bin = c - r * kHistBins;
        atomicAdd(&p.hist[(int64_t)(q0 + r0 + r) * kHistStride + bin], v);
      }
    }
  };
  auto emit = [&](int r, int pos, float sc) {
    if (pos <= first_pos + r0 + r) {
      p.scores[(int64_t)(q0 + r0 + r) * p.score_stride + pos] = sc;
      atomicAdd(&hl[r * kHistBins + (score_key(sc) >> kLevelShift[0])], 1u);
    }
  };
  enter(b);

  if (DT == 0) {
    for (int f = f0; f < f1; ++f) {
      if (f - base >= nchunks) {
        leave();
        base += nchunks;
        int nbq = b + 1;
        while (chunks_of(p, nbq, r0) == 0) ++nbq;
        enter(nbq);
      }
      const int pos = (f - base) * kChunk + tid;
      if (pos <= pos_max) {
        const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
        const float* krow = static_cast<const float*>(p.k) + ((int64_t)btrow[pos >> 6] * kPage + (pos & 63)) * D;
        score_pos_f32<D>(reinterpret_cast<const float*>(qs), wsm, p.H, nrows, krow,
                         [&](int r, float sc) { emit(r, pos, sc); });
      }
    }
  } else {
    const unsigned char* kbase = static_cast<const unsigned char*>(p.k);
    // look-ahead cursor: the request, its first flat chunk and page limit of chunk fn
    int nb_req = b, nb_base = base, nb_chunks = nchunks, nb_posmax = pos_max;
    auto advance_to = [&](int fn) {
      while (fn - nb_base >= nb_chunks) {
        nb_base += nb_chunks;
        ++nb_req;
        nb_chunks = chunks_of(p, nb_req, r0);
        if (nb_chunks) {
          const int nbb = p.q_offsets[nb_req + 1] - p.q_offsets[nb_req];
          nb_posmax = p.ctx_lens[nb_req] - nbb + r0 + min(kRowsPerBlock, nbb - r0) - 1;
        }
      }
    };
    auto load = [&](KeyTiles<DT, D, 4>& t, int phys) {
      load_key_tiles<DT, D, 4>(t, kbase + (int64_t)phys * kPage * D * Gm::ES,
                               DT == 2 ? p.k_scale + (int64_t)phys * kPage : nullptr, 0);
    };
    // block-table entry of this wave's page of chunk fn (-1: none); read one
    // chunk ahead of the tile load that needs it, so the tile loads never wait
    // on a block-table read
    auto page_of = [&](int fn) {
      if (fn >= f1) return -1;
      advance_to(fn);
      const int pgn = (fn - nb_base) * (kChunk / kPage) + wave;
      return pgn * kPage <= nb_posmax ? p.bt[(int64_t)nb_req * p.bt_stride + pgn] : -1;
    };
    KeyTiles<DT, D, 4> cur, nxt;
    bool have = false;
    {
      const int pg = (f0 - base) * (kChunk / kPage) + wave;
      if (pg * kPage <= pos_max) {
        load(nxt, p.bt[(int64_t)b * p.bt_stride + pg]);
        have = true;
      }
    }
    int ph1 = page_of(f0 + 1);
    for (int f = f0; f < f1; ++f) {
      if (f - base >= nchunks) {
        leave();
        base += nchunks;
        int nbq = b + 1;
        while (chunks_of(p, nbq, r0) == 0) ++nbq;
        enter(nbq);
      }
      cur = nxt;
      const bool have_cur = have;
      have = ph1 >= 0;
      if (have) load(nxt, ph1);  // next chunk's page for this wave
      ph1 = page_of(f + 2);
      if (have_cur) {
        const int pg = (f - base) * (kChunk / kPage) + wave;
        // one or four rows of 64 heads (decode, speculative verify) with
        // the row and head-tile loops unrolled, anything else through the
        // general loops; the sums are formed in the same order either way
        auto em = [&](int r, int slot, float sc) { emit(r, pg * kPage + slot, sc); };
        if (nrows == 4 && p.Hpad == 64)
          score_key_tiles<DT, D, 4, 4, 4>(qs, wsm, 64, 4, cur, 0, em);
        else if (nrows == 1 && p.Hpad == 64)
          score_key_tiles<DT, D, 4, 1, 4>(qs, wsm, 64, 1, cur, 0, em);
        else
          score_key_tiles<DT, D, 4>(qs, wsm, p.Hpad, nrows, cur, 0, em);
      }
    }
  }
  leave();
}

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kCandCap = 12288;
constexpr int kItems = 4;  // consecutive positions per thread per pass

struct TopkParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  int batch;
  const float* scores;
  int64_t score_stride;
  uint32_t* hist;
  int K;
  int32_t* out;
  int only_flagged;  // handle only the rows the segment kernels left (flag word set)
};

struct TopkShared {
  uint32_t bins[kHistBins];
  uint32_t cand[kCandCap];
  alignas(16) int wsum[kTopkThreads / 64];
  int ncand;
  int res_bin, res_above;
};

__device__ __forceinline__ void load_keys(const float* row, int t0, int vis, uint32_t key[kItems],
                                          bool valid[kItems]) {
  if (t0 + kItems <= vis) {
    const float4 v = *reinterpret_cast<const float4*>(row + t0);
    key[0] = score_key(v.x); key[1] = score_key(v.y); key[2] = score_key(v.z); key[3] = score_key(v.w);
#pragma unroll
    for (int e = 0; e < kItems; ++e) valid[e] = true;
  } else {
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      valid[e] = (t0 + e) < vis;
      key[e] = valid[e] ? score_key(row[t0 + e]) : 0u;
    }
  }
}

// Wave 0 finds the bin; the result is broadcast through LDS.
__device__ __forceinline__ void kth_bin_block(TopkShared& sh, int nbins, int k) {
  if (threadIdx.x < 64) {
    int bin, above;
    kth_bin_wave(sh.bins, nbins, k, bin, above);
    if (threadIdx.x == 0) {
      sh.res_bin = bin;
      sh.res_above = above;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(kTopkThreads) void li_topk(TopkParams p) {
  __shared__ TopkShared sh;
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int nb = p.q_offsets[b + 1] - p.q_offsets[b];
  const int vis = p.ctx_lens[b] - nb + (i - p.q_offsets[b]) + 1;
  const int K = p.K;
  int32_t* out = p.out + (int64_t)i * K;
  uint32_t* hrow = p.hist + (int64_t)i * kHistStride;
  if (p.only_flagged && (vis <= K || hrow[kHistStride - 1] != 1u)) return;
  if (vis <= K) {  // everything visible is kept
    for (int t = tid; t < K; t += kTopkThreads) out[t] = t < vis ? t : -1;
    for (int c = tid; c < kHistBins; c += kTopkThreads) hrow[c] = 0u;
    return;
  }
  const float* row = p.scores + (int64_t)i * p.score_stride;

  // level 1 from the scoring kernel's histogram, which is then cleared
  for (int c = tid; c < kHistBins; c += kTopkThreads) {
    sh.bins[c] = hrow[c];
    hrow[c] = 0u;
  }
  if (tid == 0) sh.ncand = 0;
  __syncthreads();
  kth_bin_block(sh, kHistBins, K);
  const uint32_t bin1 = sh.res_bin;
  int need = K - sh.res_above;  // keys still needed from bin1 (>= 1)
  const bool in_lds = sh.bins[bin1] <= (uint32_t)kCandCap;
  __syncthreads();

  // gather bin1's keys (low 21 bits) into LDS when they fit
  if (in_lds) {
    for (int t0 = tid * kItems; t0 < vis; t0 += kTopkThreads * kItems) {
      uint32_t key[kItems];
      bool valid[kItems];
      load_keys(row, t0, vis, key, valid);
#pragma unroll
      for (int e = 0; e < kItems; ++e) {
        const bool pred = valid[e] && (key[e] >> 21) == bin1;
        const uint64_t m = __ballot(pred);
        const int n = __popcll(m);
        int base = 0;
        if (n) {
          if (lane == 0) base = atomicAdd(&sh.ncand, n);
          base = wave_read_lane(base, 0);  // lane 0 is active whenever any lane is
        }
        const int slot = base + __popcll(m & ((1ull << lane) - 1ull));
        if (pred && slot < kCandCap) sh.cand[slot] = key[e] & 0x1fffffu;
      }
    }
    __syncthreads();
  }
  const int ncand = in_lds ? min(sh.ncand, kCandCap) : 0;

  // levels 2 (key bits 20..10) and 3 (bits 9..0) over bin1's keys
  uint32_t prefix = bin1;  // known high bits of the K-th key
  for (int level = 1; level < 3; ++level) {
    const int nbins = kLevelBins[level];
    const int shift = kLevelShift[level];
    for (int c = tid; c < nbins; c += kTopkThreads) sh.bins[c] = 0u;
    __syncthreads();
    if (in_lds) {
      for (int c = tid; c < ncand; c += kTopkThreads) {
        const uint32_t low = sh.cand[c];
        if (level == 1 || (low >> 10) == (prefix & 2047u)) atomicAdd(&sh.bins[(low >> shift) & (nbins - 1)], 1u);
      }
    } else {
      for (int t0 = tid * kItems; t0 < vis; t0 += kTopkThreads * kItems) {
        uint32_t key[kItems];
        bool valid[kItems];
        load_keys(row, t0, vis, key, valid);
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
          const bool hit = valid[e] && (key[e] >> kLevelShift[level - 1]) == prefix;
          if (hit) atomicAdd(&sh.bins[(key[e] >> shift) & (nbins - 1)], 1u);
        }
      }
    }
    __syncthreads();
    kth_bin_block(sh, nbins, need);
    prefix = (prefix << (level == 1 ? 11 : 10)) | (uint32_t)sh.res_bin;
    need -= sh.res_above;
    __syncthreads();
  }
  const uint32_t kth = prefix;  // the K-th largest key; `need` keys equal to it are kept

  // ordered pass: keep keys > kth and the first `need` keys == kth (lowest positions)
  int eq_run = 0, written = 0;
  for (int base = 0; base < vis && written < K; base += kTopkThreads * kItems) {
    const int t0 = base + tid * kItems;
    uint32_t key[kItems];
    bool valid[kItems];
    if (t0 < vis) {
      load_keys(row, t0, vis, key, valid);
    } else {
#pragma unroll
      for (int e = 0; e < kItems; ++e) {
        valid[e] = false;
        key[e] = 0u;
      }
    }
    int neq = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) neq += (valid[e] && key[e] == kth);
    int eq_total;
    int eq_before = block_excl_scan<kTopkThreads>(neq, eq_total, sh.wsum) + eq_run;
    bool sel[kItems];
    int nsel = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      const bool is_eq = valid[e] && key[e] == kth;
      sel[e] = (valid[e] && key[e] > kth) || (is_eq && eq_before < need);
      eq_before += is_eq;
      nsel += sel[e];
    }
    int sel_total;
    int pos = block_excl_scan<kTopkThreads>(nsel, sel_total, sh.wsum) + written;
#pragma unroll
    for (int e = 0; e < kItems; ++e)
      if (sel[e] && pos < K) out[pos++] = t0 + e;
    eq_run += eq_total;
    written += sel_total;
  }
  for (int t = written + tid; t < K; t += kTopkThreads) out[t] = -1;  // only on inconsistent input
}

}  // namespace dsa

using namespace dsa;

template <typename Kern, typename P>
static hipError_t launch_dyn(Kern kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const P& p) {
  {
    const hipError_t e = dsa_allow_lds(reinterpret_cast<const void*>(kernel), lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, s, p);
  return hipGetLastError();
}

template <int DT, int D>
static hipError_t launch_score(const LiParams& p, dim3 grid, hipStream_t s) {
  const size_t lds = query_lds_bytes<DT, D>(p.rcap, p.Hpad) + (size_t)p.rcap * kHistBins * 4;
  return launch_dyn(li_score<DT, D>, grid, dim3(kScoreThreads), lds, s, p);
}

hipError_t dsa_launch_indexer_scores(const DsaIndexerLaunch& a, hipStream_t s) {
  LiParams p;
  p.q_offsets = a.q_offsets;
  p.ctx_lens = a.ctx_lens;
  p.bt = a.block_table;
  p.batch = a.batch;
  p.bt_stride = a.bt_stride;
  p.H = a.n_heads;
  p.Hpad = a.dtype == 0 ? a.n_heads : ((a.n_heads + 15) / 16) * 16;
  p.rcap = std::min(kRowsPerBlock, a.max_q_per_req);
  p.q = a.q;
  p.q_scale = a.q_scale;
  p.w = a.weights;
  p.k = a.k_cache;
  p.k_scale = a.k_scale;
  p.scores = a.scores;
  p.score_stride = a.score_stride;
  p.hist = a.hist;

  hipError_t e;
  if (dsa_indexer_rows_route(a)) {
    e = dsa_launch_indexer_prefill_scores(a, s);
  } else {
    // one list of chunks over all requests per row group, split over gx workgroups
    const int chunks = (a.max_ctx_len + kChunk - 1) / kChunk;
    const int gx = (int)std::max<int64_t>(1, std::min<int64_t>(kScoreTargetWGs, (int64_t)chunks * a.batch));
    const dim3 grid(gx, (a.max_q_per_req + kRowsPerBlock - 1) / kRowsPerBlock);
    const bool d64 = a.head_dim == 64;
    switch (a.dtype) {
      case 0: e = d64 ? launch_score<0, 64>(p, grid, s) : launch_score<0, 128>(p, grid, s); break;
      case 1: e = d64 ? launch_score<1, 64>(p, grid, s) : launch_score<1, 128>(p, grid, s); break;
      default: e = d64 ? launch_score<2, 64>(p, grid, s) : launch_score<2, 128>(p, grid, s); break;
    }
  }
  return e;
}

hipError_t dsa_launch_indexer_two_pass(const DsaIndexerLaunch& a, hipStream_t s) {
  hipError_t e = dsa_launch_indexer_scores(a, s);
  if (e != hipSuccess) return e;

  e = dsa_launch_topk_segments(a, s);
  if (e != hipSuccess) return e;
  // rows whose boundary bin overflowed the candidate list
  TopkParams tp;
  tp.q_offsets = a.q_offsets;
  tp.ctx_lens = a.ctx_lens;
  tp.batch = a.batch;
  tp.scores = a.scores;
  tp.score_stride = a.score_stride;
  tp.hist = a.hist;
  tp.K = a.topk;
  tp.out = a.out_idx;
  tp.only_flagged = 1;
  hipLaunchKernelGGL(li_topk, dim3(a.num_rows), dim3(kTopkThreads), 0, s, tp);
  return hipGetLastError();
}
