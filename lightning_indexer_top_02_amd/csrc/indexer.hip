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
// Selection runs over segments of each row (topk_seg.hip).
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
  const void* q_scale;
  const float* w;
  const void* k;
  const void* k_scale;
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
                               page_scales<DT, D>(p.k_scale, phys), 0);
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
      case 2: e = d64 ? launch_score<2, 64>(p, grid, s) : launch_score<2, 128>(p, grid, s); break;
      default: e = launch_score<3, 128>(p, grid, s); break;  // MXFP8: 128-dim only
    }
  }
  return e;
}

hipError_t dsa_launch_indexer_two_pass(const DsaIndexerLaunch& a, hipStream_t s) {
  hipError_t e = dsa_launch_indexer_scores(a, s);
  if (e != hipSuccess) return e;

  return dsa_launch_topk_segments(a, s);
}
