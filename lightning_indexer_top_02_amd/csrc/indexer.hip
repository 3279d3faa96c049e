// indexer.hip -- lightning indexer, throughput path (gfx950): scores through
// HBM, then the segment-parallel selection of topk_seg.hip.
//
// Used when rows are too long (or too many per request) for the single fused
// kernel (indexer_fused.hip).  Requests with many query rows (chunked
// prefill) are scored by the row-tiled MFMA kernel of indexer_prefill.hip
// instead of li_score; both write the same scores and histograms.  The
// scoring follows "Optimizing Inference for Hybrid Attention Architectures:
// From Operator Fusion to Sequence Sharding", section "Breaking Down the
// Computational Path of Hybrid Attention", item 1, reading keys straight from
// the paged K cache ("Day0 Inference Support and Performance Optimization for
// New LLM Architectures", section III, 3.1).
//
// li_score: one workgroup = 4 waves, stepping 4 cache pages (256 positions)
// at a time through its share of all requests' chunks, for up to 4 query rows
// of the request at hand (the rows share one read of the keys).
// It writes fp32 scores and a per-row histogram of the top 11 key bits (LDS,
// then one global atomic per non-empty bin): the first radix level.
#include <algorithm>
#include <type_traits>

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
// Chunks whose block-table entries a workgroup stages in LDS at a time.
constexpr int kWinChunks = 256;

// Chunks of 256 positions row group y (rows 4y .. 4y + 3) of request b
// covers: every position its last row sees, 0 when the request has no such
// rows.
__device__ __forceinline__ int chunks_of(const LiParams& p, int b, int r0) {
  const int nb = p.q_offsets[b + 1] - p.q_offsets[b];
  if (r0 >= nb) return 0;
  const int pos_max = p.ctx_lens[b] - nb + r0 + min(kRowsPerBlock, nb - r0) - 1;
  return pos_max / kChunk + 1;
}

template <int DT, int D>
__host__ __device__ constexpr size_t score_lds_bytes(int rcap, int Hpad) {
  return query_lds_bytes<DT, D>(rcap, Hpad) + (size_t)rcap * kHistBins * 4 + (DT == 0 ? 0 : kWinChunks * 4 * 4);
}

// The chunks of all requests (for one row group) form one list, split evenly
// over the workgroups of the grid's x dimension, so requests of different
// lengths cost their share and no workgroup waits on a long one.  A
// workgroup walks its range request by request: it stages the request's
// query rows (and starts its histogram), scores its chunks of the request,
// and flushes the histogram.  For bf16 and fp8 keys the block-table entries
// of up to 256 chunks go to LDS first, then each wave scores its page of
// every chunk with its next page's tiles in flight (1-byte keys: the next
// two pages', three tile sets rotating).  Every chunk issues the same vector
// memory operations: past the range a valid page is loaded and not used,
// pages past the rows' last position are scored and not stored, and the
// score stores are buffer stores whose masked lanes carry an offset the
// hardware drops.  The wait for a tile set therefore leaves the later sets'
// loads in flight (a conditional store or load among them would make it wait
// for everything).
template <int DT, int D>
__global__ __launch_bounds__(kScoreThreads, 2) __attribute__((amdgpu_waves_per_eu(2, 2))) void li_score(LiParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ __align__(16) int wsum[kScoreThreads / 64];
  __shared__ int s_b0, s_base0;
  using Gm = IdxGeom<DT, D>;
  unsigned char* qs = smem;
  float* wsm = reinterpret_cast<float*>(smem + (size_t)p.rcap * p.Hpad * Gm::QSTRIDE);
  uint32_t* hl = reinterpret_cast<uint32_t*>(wsm + p.rcap * p.Hpad);
  int* pages = reinterpret_cast<int*>(hl + p.rcap * kHistBins);  // [kWinChunks][4] (bf16 / fp8)
  const int tid = threadIdx.x, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
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

  // the request being scored (uniform over the workgroup)
  int b = __builtin_amdgcn_readfirstlane(s_b0), base = __builtin_amdgcn_readfirstlane(s_base0);
  int q0 = 0, nrows = 0, first_pos = 0, pos_max = -1, nchunks = 0;
  __amdgpu_buffer_rsrc_t srs;  // this request's row group of the score rows
  auto enter = [&]() {
    q0 = p.q_offsets[b];
    const int nb = p.q_offsets[b + 1] - q0;
    nrows = min(kRowsPerBlock, nb - r0);
    first_pos = p.ctx_lens[b] - nb;
    pos_max = first_pos + r0 + nrows - 1;
    nchunks = pos_max / kChunk + 1;
    srs = __builtin_amdgcn_make_buffer_rsrc(p.scores + (int64_t)(q0 + r0) * p.score_stride, 0,
                                            (int)((int64_t)nrows * p.score_stride * 4), 0x00020000);
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
  // Every lane issues the store; a position row r does not see gets an
  // offset past the buffer, which the hardware drops.
  auto emit = [&](int r, int pos, float sc) {
    const bool ok = pos <= first_pos + r0 + r;
    const uint32_t off = ok ? (uint32_t)(r * p.score_stride + pos) * 4u : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(sc), srs, (int)off, 0, 0);
    asm volatile("" ::: "memory");  // (keeps the store out of the branch below)
    if (ok) atomicAdd(&hl[r * kHistBins + (score_key(sc) >> kLevelShift[0])], 1u);
  };

  const unsigned char* kbase = static_cast<const unsigned char*>(p.k);
  int f = f0;
  while (true) {
    enter();
    const int c_begin = f - base, c_end = min(f1 - base, nchunks);  // chunks of this request here
    if constexpr (DT == 0) {
      const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
      for (int c = c_begin; c < c_end; ++c) {
        const int pos = c * kChunk + tid;
        if (pos <= pos_max) {
          const float* krow = static_cast<const float*>(p.k) + ((int64_t)btrow[pos >> 6] * kPage + (pos & 63)) * D;
          score_pos_f32<D>(reinterpret_cast<const float*>(qs), wsm, p.H, nrows, krow,
                           [&](int r, float sc) { emit(r, pos, sc); });
        }
      }
    } else {
      const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
      for (int w0 = c_begin; w0 < c_end; w0 += kWinChunks) {
        const int n = min(kWinChunks, c_end - w0);
        // block-table entries of the window: entry 4j + i is page i of chunk
        // w0 + j, or the window's first page past the rows' last position
        __syncthreads();
        for (int i = tid; i < 4 * n; i += kScoreThreads) {
          const int pg = w0 * 4 + i;
          pages[i] = btrow[pg * kPage <= pos_max ? pg : w0 * 4];
        }
        __syncthreads();
        auto load = [&](KeyTiles<DT, D, 4>& t, int j) __attribute__((always_inline)) {
          // this wave's page of chunk w0 + j (clamped), in a scalar register:
          // the addresses are then a scalar base plus fixed lane offsets, and
          // no vector register is written between a tile's loads and its use
          const int phys = __builtin_amdgcn_readfirstlane(pages[4 * min(j, n - 1) + wave_u]);
          load_key_tiles<DT, D, 4>(t, kbase + (int64_t)phys * kPage * D * Gm::ES,
                                   page_scales<DT, D>(p.k_scale, phys), 0);
          // issued here, not sunk below the scoring that follows (the
          // scheduler would otherwise reuse the scored tile's registers)
          __builtin_amdgcn_sched_barrier(0);
        };
        // The ring for one scoring shape: one or four rows of 64 heads
        // (decode, speculative verify) and one row of at most 16 heads (the
        // narrow indexer) with the row and head-tile loops unrolled, anything
        // else through the general loops (the sums are
        // formed in the same order either way).  Everything is inlined so the
        // tile sets stay in registers.
        auto ring_loop = [&](auto nr_c, auto mt_c) __attribute__((always_inline)) {
          constexpr int NR = decltype(nr_c)::value, MT = decltype(mt_c)::value;
          auto score = [&](const KeyTiles<DT, D, 4>& t, int j) __attribute__((always_inline)) {
            const int pg0 = ((w0 + j) * 4 + wave_u) * kPage;
            score_key_tiles<DT, D, 4, NR, MT>(qs, wsm, MT > 0 ? 16 * MT : p.Hpad, nrows, t, 0,
                                              [&](int r, int slot, float sc) { emit(r, pg0 + slot, sc); });
          };
          if constexpr (Gm::ES == 1 && NR > 0) {  // 1-byte keys, unrolled shapes: two tile sets ahead
            KeyTiles<DT, D, 4> t0, t1, t2;
            load(t0, 0);
            load(t1, 1);
            // whole turns of the ring, then the one or two chunks left: no
            // exit inside the loop, so the waits in it see only the ring's
            // own loads in flight
            int j = 0;
            for (; j + 3 <= n; j += 3) {
              load(t2, j + 2);
              score(t0, j);
              load(t0, j + 3);
              score(t1, j + 1);
              load(t1, j + 4);
              score(t2, j + 2);
            }
            if (j < n) score(t0, j);
            if (j + 1 < n) score(t1, j + 1);
          } else {
            KeyTiles<DT, D, 4> t0, t1;
            load(t0, 0);
            int j = 0;
            for (; j + 2 <= n; j += 2) {
              load(t1, j + 1);
              score(t0, j);
              load(t0, j + 2);
              score(t1, j + 1);
            }
            if (j < n) score(t0, j);
          }
        };
        if (nrows == 4 && p.Hpad == 64)
          ring_loop(std::integral_constant<int, 4>{}, std::integral_constant<int, 4>{});
        else if (nrows == 1 && p.Hpad == 64)
          ring_loop(std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{});
        else if (nrows == 1 && p.Hpad == 16)
          ring_loop(std::integral_constant<int, 1>{}, std::integral_constant<int, 1>{});
        else
          ring_loop(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
      }
    }
    leave();
    f = base + c_end;
    if (f >= f1) break;
    base += nchunks;
    do {
      ++b;
    } while (chunks_of(p, b, r0) == 0);
    b = __builtin_amdgcn_readfirstlane(b);
  }
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
  // buffer-store offsets are 32-bit: a row group's scores must stay below 2 GiB
  if ((int64_t)kRowsPerBlock * p.score_stride * 4 >= (int64_t)1 << 31) return hipErrorInvalidValue;
  return launch_dyn(li_score<DT, D>, grid, dim3(kScoreThreads), score_lds_bytes<DT, D>(p.rcap, p.Hpad), s, p);
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
