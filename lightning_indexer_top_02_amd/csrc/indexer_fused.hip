// indexer_fused.hip -- lightning indexer, latency path (gfx950): scoring,
// head weighting and Top-K selection in one kernel launch.
//
// The pages fuse the three indexer steps into one operator that reads the
// paged K cache directly and outputs only the Top-K indices ("Day0 Inference
// Support and Performance Optimization for New LLM Architectures", section
// III, 3.1; "Optimizing Inference for Hybrid Attention Architectures: From
// Operator Fusion to Sequence Sharding", section "Fusing Index Screening with
// Multi-Stream Orchestration").  On one MI355X a single decode row is too
// short for one workgroup to stream at HBM speed, and measured cross-XCD
// synchronisation inside a kernel costs tens of microseconds per round (every
// workgroup of a team re-reading one shared histogram), so this kernel never
// waits:
//   * the G workgroups of a request score its positions in chunks of 256
//     (one 16-position MFMA tile per wave), chunk m, m + G, ... for workgroup
//     m, for all of that request's query rows, and write the scores as
//     order-preserving 32-bit keys to the workspace (G = all chunks for a
//     single request; fewer, each looping, for a batch);
//   * each workgroup adds its share of each row's histogram of the top 11
//     key bits to the workspace and counts itself done on the request's
//     arrival counter; the last workgroup to arrive loads each row's keys
//     (at most 32768, 32 per thread) into registers, takes the first digit
//     of the K-th key from the finished histogram and runs the two remaining
//     radix digits and the ordered write there (select_from_level1).
// The keys make one round trip through the L2/Infinity Cache (4 bytes per
// position against the 128-256 bytes of key read per position).  Rows longer
// than 32768 positions take the two-pass route (indexer.hip).
#include <algorithm>

#include "dsa_device.h"
#include "indexer_common.h"
#include "radix_select.h"

namespace dsa {

struct FusedParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* bt;
  int batch, bt_stride;
  int H, Hpad, rcap;
  const void* q;
  const void* q_scale;
  const float* w;
  const void* k;
  const void* k_scale;
  int K;
  int32_t* out;
  int G;                // workgroups per request (each takes every G-th chunk)
  int row_cap;          // min(max_ctx_len, kFusedMaxRow)
  uint32_t* keys;       // [rows][key_stride] score keys
  int64_t key_stride;
  uint32_t* counters;   // [batch] arrival counters, zero between calls
  uint32_t* hist;       // [rows][kHistStride]: top-11-bit key histogram at offset 0, zero between calls
  int kbuf_stride;      // > 0: keys are staged in LDS, this many per row (0: stored as they are made)
};

constexpr int kFusedThreads = 1024;
constexpr int kFusedWaves = kFusedThreads / 64;
constexpr int kFusedChunk = kFusedWaves * 16;  // positions per workgroup
constexpr int kFusedMaxRow = 32768;            // longest row the selection holds in LDS
constexpr int kFusedMaxRows = 4;               // query rows per request
constexpr int kKeysPerThread = kFusedMaxRow / kFusedThreads;
constexpr int kFusedMaxPages = kFusedMaxRow / kFusedChunk * (kFusedChunk / kPage);  // pages one workgroup scores
constexpr int kFusedKeyBuf = 16384;  // keys a workgroup may stage in LDS (64 KB)
constexpr size_t kLdsPerWorkgroup = 160 * 1024;  // gfx950
constexpr size_t kFusedStaticLds = 256;           // wsum, res and s_last, rounded up

// Slot of position p in a row's key array.  The selecting workgroup holds
// positions 32 t .. 32 t + 31 in thread t and loads them 4 at a time; keys
// are stored in groups of 4 positions, transposed so that group j of every
// thread is contiguous: slot = j S + 4 t + p % 4 with j = (p % 32) / 4,
// t = p / 32 and S = 4 ceil(row_cap / 32).  Those loads are then coalesced
// (a wave reads 1 KB in one piece instead of 64 lines 128 bytes apart).
__device__ __forceinline__ int key_slot(int p, int S) { return ((p & 31) >> 2) * S + ((p >> 5) << 2) + (p & 3); }

// MODE 0: few chunks per workgroup (small batches): latency first.
// MODE 1: many chunks per workgroup: block-table entries in LDS, three key
//         tiles in rotation, keys staged in LDS and written out at the end.
// MODE 2: MODE 1 where every request has one query row and 64 heads (the
//         decode shape): the scoring has no inner loops over rows and head
//         tiles, which keeps the prefetched key tiles in flight.
template <int DT, int D, int MODE>
__global__ __launch_bounds__(kFusedThreads) void li_fused(FusedParams p) {
  using Gm = IdxGeom<DT, D>;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ __align__(16) int wsum[kFusedWaves];
  __shared__ int res[3];
  __shared__ int s_last;

  const int G = p.G, K = p.K;
  const int b = blockIdx.x / G, m = blockIdx.x - b * G;
  const int q0 = p.q_offsets[b], nb = p.q_offsets[b + 1] - q0;
  const int first_pos = p.ctx_lens[b] - nb;  // position of the request's first query row
  const int pos_max = first_pos + nb - 1;    // last position any of its rows sees
  const int c0 = m * kFusedChunk;
  const int tid = threadIdx.x, wave = tid >> 6;
  const bool any_select = pos_max + 1 > K;   // the last row sees the most positions
  const int key_group_stride = 4 * ((p.row_cap + 31) / 32);

  // ---- scoring: one 16-position tile per wave per chunk ----------------------
  // Workgroup m of a request takes chunks m, m + G, m + 2G, ... (G is chosen
  // so the whole batch gives a few workgroups per compute unit); the next
  // chunk's key tile is loaded before the current one is scored.
  if (any_select && c0 <= pos_max) {
    unsigned char* qs = smem;
    float* wsm = reinterpret_cast<float*>(smem + (size_t)p.rcap * p.Hpad * Gm::QSTRIDE);
    // this workgroup's share of each row's histogram of the top 11 key bits
    uint32_t* lh = reinterpret_cast<uint32_t*>(smem + query_lds_bytes<DT, D>(p.rcap, p.Hpad));
    const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
    const unsigned char* kbase = static_cast<const unsigned char*>(p.k);
    const int step = G * kFusedChunk;
    int* wg_pages = reinterpret_cast<int*>(smem + query_lds_bytes<DT, D>(p.rcap, p.Hpad) +
                                           (size_t)p.rcap * kHistBins * 4);
    uint32_t* kbuf = reinterpret_cast<uint32_t*>(wg_pages + kFusedMaxPages);
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    int t0 = c0 + wave_u * 16;
    const int last_j = t0 <= pos_max ? (pos_max - t0) / step : -1;  // this wave's last chunk
    KeyTiles<DT, D, 1> ring[3];
    auto load_at = [&](KeyTiles<DT, D, 1>& t, int phys, int tpos) {
      load_key_tiles<DT, D, 1>(t, kbase + (int64_t)phys * kPage * D * Gm::ES,
                               page_scales<DT, D>(p.k_scale, phys), tpos & 63);
    };
    if constexpr (MODE == 0) {
      // few chunks per workgroup (small batches): the first key tile is in
      // flight while the queries are staged
      if (DT != 0 && last_j >= 0) load_at(ring[0], btrow[t0 >> 6], t0);
    } else {
      // Many chunks per workgroup: the block-table entries of every page it
      // scores go to LDS first (entry 4 j + i: page i of its j-th chunk), so a
      // key tile's load waits only on LDS, never on the vector loads of the
      // tiles in flight.  Three key tiles rotate: two chunks ahead are in
      // flight while one is scored.  Every step issues its loads (past the
      // wave's last chunk, that chunk again), so the wait for a tile always
      // has the two later tiles' loads behind it and leaves them in flight.
      const int n_pages = ((pos_max - c0) / step + 1) * (kFusedChunk / kPage);
      for (int i = tid; i < n_pages; i += kFusedThreads) {
        const int pg = c0 / kPage + (i / (kFusedChunk / kPage)) * (step / kPage) + i % (kFusedChunk / kPage);
        wg_pages[i] = pg <= pos_max / kPage ? btrow[pg] : 0;
      }
      __syncthreads();
      if (last_j >= 0) {
        load_at(ring[0], wg_pages[wave_u / (kPage / 16)], t0);
        load_at(ring[1], wg_pages[min(1, last_j) * (kFusedChunk / kPage) + wave_u / (kPage / 16)], t0);
      }
    }
    stage_queries<DT, D, kFusedThreads>(qs, wsm, p.q, p.q_scale, p.w, q0, nb, p.H, p.Hpad);
    for (int c = tid; c < nb * kHistBins; c += kFusedThreads) lh[c] = 0u;
    __syncthreads();
    // In the batched modes keys go to LDS when they fit (chunk j's 256 keys
    // at j * 256 of the row's stretch) and are written out in whole lines
    // once the workgroup is done: stores among the scoring loads would make
    // every wait for a key tile also wait for them.
    auto emit = [&](int r, int pos, float s) {
      if (pos <= first_pos + r) {
        const uint32_t k = score_key(s);
        if (MODE != 0 && p.kbuf_stride > 0) {
          const int j = (pos - c0) / step;
          kbuf[r * p.kbuf_stride + j * kFusedChunk + (pos - c0 - j * step)] = k;
        } else {
          p.keys[(int64_t)(q0 + r) * p.key_stride + key_slot(pos, key_group_stride)] = k;
        }
        atomicAdd(&lh[r * kHistBins + (k >> kLevelShift[0])], 1u);
      }
    };
    if (DT == 0) {
      const int lane = tid & 63;
      for (int c = c0; c <= pos_max; c += step) {
        const int tp = c + wave * 16;
        if (lane < 16 && tp + lane <= pos_max) {
          const int pos = tp + lane;
          const float* krow = static_cast<const float*>(p.k) + ((int64_t)btrow[pos >> 6] * kPage + (pos & 63)) * D;
          score_pos_f32<D>(reinterpret_cast<const float*>(qs), wsm, p.H, nb, krow,
                           [&](int r, float s) { emit(r, pos, s); });
        }
      }
    } else if constexpr (MODE == 0) {
      for (; t0 <= pos_max; t0 += step) {
        ring[1] = ring[0];
        if (t0 + step <= pos_max) load_at(ring[0], btrow[(t0 + step) >> 6], t0 + step);
        score_key_tiles<DT, D, 1>(qs, wsm, p.Hpad, nb, ring[1], t0 & 63,
                                  [&](int r, int slot, float s) { emit(r, (t0 & ~63) + slot, s); });
      }
    } else {
      auto load = [&](KeyTiles<DT, D, 1>& t, int j) {  // this wave's tile of chunk j
        load_at(t, wg_pages[j * (kFusedChunk / kPage) + wave_u / (kPage / 16)], t0);
      };
      auto score = [&](const KeyTiles<DT, D, 1>& kt, int tc) {
        auto em = [&](int r, int slot, float s) { emit(r, (tc & ~63) + slot, s); };
        if constexpr (MODE == 2)  // one row of 64 heads: no inner loops
          score_key_tiles<DT, D, 1, 1, 4>(qs, wsm, 64, 1, kt, tc & 63, em);
        else
          score_key_tiles<DT, D, 1>(qs, wsm, p.Hpad, nb, kt, tc & 63, em);
      };
      for (int j = 0; j <= last_j; j += 3) {
        load(ring[2], min(j + 2, last_j));
        score(ring[0], t0 + j * step);
        if (j + 1 > last_j) break;
        load(ring[0], min(j + 3, last_j));
        score(ring[1], t0 + (j + 1) * step);
        if (j + 2 > last_j) break;
        load(ring[1], min(j + 4, last_j));
        score(ring[2], t0 + (j + 2) * step);
      }
    }
  }

  // ---- staged keys and the histograms go to the workspace (the histogram
  // sums are complete when the last workgroup arrives)
  if (any_select && c0 <= pos_max) {
    const uint32_t* lh = reinterpret_cast<const uint32_t*>(smem + query_lds_bytes<DT, D>(p.rcap, p.Hpad));
    __syncthreads();
    if (MODE != 0 && p.kbuf_stride > 0) {
      // item i: row r, chunk j, line L of the chunk's 8 slot lines, word k;
      // 32 consecutive items fill one 128-byte line of the key array
      const int step = G * kFusedChunk;
      const int n_ch = (pos_max - c0) / step + 1;
      const uint32_t* kbuf = reinterpret_cast<const uint32_t*>(smem + query_lds_bytes<DT, D>(p.rcap, p.Hpad) +
                                                               (size_t)p.rcap * kHistBins * 4 + kFusedMaxPages * 4);
      for (int i = tid; i < nb * n_ch * kFusedChunk; i += kFusedThreads) {
        const int r = i / (n_ch * kFusedChunk), rest = i - r * n_ch * kFusedChunk;
        const int j = rest / kFusedChunk, w = rest - j * kFusedChunk;
        const int L = w >> 5, k = w & 31;
        const int cs = c0 + j * step;                 // the chunk's first position
        const int pos = cs + 32 * (k >> 2) + 4 * L + (k & 3);
        if (pos <= first_pos + r)
          p.keys[(int64_t)(q0 + r) * p.key_stride + key_slot(pos, key_group_stride)] =
              kbuf[r * p.kbuf_stride + j * kFusedChunk + (pos - cs)];
      }
    }
    for (int c = tid; c < nb * kHistBins; c += kFusedThreads) {
      const uint32_t v = lh[c];
      if (v) {
        const int r = c / kHistBins;
        atomicAdd(&p.hist[(int64_t)(q0 + r) * kHistStride + (c - r * kHistBins)], v);
      }
    }
  }

  // ---- arrival: the last workgroup of the request selects ---------------------
  // Each thread waits for its own key stores; one agent-scope release per
  // workgroup then publishes them (a device-wide fence in every thread costs
  // tens of microseconds at this grid size).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    if (!any_select) {
      s_last = m == 0;  // nothing to rank: workgroup 0 writes the outputs
    } else {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      const uint32_t old = __hip_atomic_fetch_add(p.counters + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = old == (uint32_t)G - 1;
      if (s_last) {
        __hip_atomic_store(p.counters + b, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // see every other workgroup's keys
      }
    }
  }
  __syncthreads();
  if (!s_last) return;

  uint32_t* hist = reinterpret_cast<uint32_t*>(smem);  // the query staging area is free now
  for (int r = 0; r < nb; ++r) {
    const int vis = first_pos + r + 1;
    int32_t* out = p.out + (int64_t)(q0 + r) * K;
    if (vis <= K) {
      for (int t = tid; t < K; t += kFusedThreads) out[t] = t < vis ? t : -1;
      continue;
    }
    // the row's histogram (two bins per thread, on their way to LDS) and its
    // keys in registers (kKeysPerThread consecutive ones per thread), all
    // loads in flight together
    static_assert(kHistBins == 2 * kFusedThreads, "two histogram bins per thread");
    const uint2 hbins = reinterpret_cast<const uint2*>(p.hist + (int64_t)(q0 + r) * kHistStride)[tid];
    const uint32_t* grow = p.keys + (int64_t)(q0 + r) * p.key_stride;
    const int pos0 = tid * kKeysPerThread;
    uint32_t key[kKeysPerThread];
#pragma unroll
    for (int c = 0; c < kKeysPerThread; c += 4) {
      const int t = pos0 + c;
      const uint32_t* g4 = grow + key_slot(t, key_group_stride);
      if (t + 4 <= vis) {
        const uint4 v = *reinterpret_cast<const uint4*>(g4);
        key[c] = v.x;
        key[c + 1] = v.y;
        key[c + 2] = v.z;
        key[c + 3] = v.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) key[c + j] = t + j < vis ? g4[j] : 0u;
      }
    }
    // the first digit of the K-th key from the row's whole histogram
    reinterpret_cast<uint2*>(hist)[tid] = hbins;
    __syncthreads();
    if (wave == 0) {
      int bin, above, total;
      kth_bin_wave<kHistBins / 64>(hist, K, bin, above, total);
      if ((tid & 63) == 0) {
        res[0] = bin;
        res[1] = above;
      }
    }
    __syncthreads();
    const uint32_t bin1 = (uint32_t)res[0];
    const int need = K - res[1];
    __syncthreads();
    select_from_level1<kFusedThreads, kKeysPerThread>(key, vis, K, bin1, need, out, hist, wsum, res);
  }
  // leave every row's histogram zero for the next call
  for (int c = tid; c < nb * kHistBins; c += kFusedThreads) {
    const int r = c / kHistBins;
    p.hist[(int64_t)(q0 + r) * kHistStride + (c - r * kHistBins)] = 0u;
  }
}

}  // namespace dsa

using namespace dsa;

namespace {

// Workgroups a batch should fill: one per compute unit (a 1024-thread
// workgroup at ~128 VGPRs per thread fills one; a larger grid only queues a
// second round behind the first: 157 us against 139 us for 64 rows at 32K).
constexpr int kFusedTargetWGs = 256;

template <int DT, int D, int MODE>
hipError_t launch_fused_as(const FusedParams& p, int batch, size_t lds, hipStream_t s) {
  {
    const hipError_t e = dsa_allow_lds(reinterpret_cast<const void*>(li_fused<DT, D, MODE>), lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((li_fused<DT, D, MODE>), dim3(p.G * batch), dim3(kFusedThreads), lds, s, p);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_fused(FusedParams p, int batch, int max_ctx, hipStream_t s) {
  const int chunks = (max_ctx + kFusedChunk - 1) / kFusedChunk;
  p.G = std::max(1, std::min(chunks, (kFusedTargetWGs + batch - 1) / batch));
  p.row_cap = std::min(max_ctx, kFusedMaxRow);
  // chunks per workgroup decide the mode: with one or two the scoring is one
  // latency chain; with more, throughput (prefetch depth, no stores among
  // the loads) decides
  const int max_ch = (chunks + p.G - 1) / p.G;
  const int mode = max_ch < 3 ? 0 : (DT != 0 && p.rcap == 1 && p.Hpad == 64 ? 2 : 1);
  // batched modes stage a workgroup's keys in LDS when they fit, both the
  // staging cap and the device's LDS beside the queries, histograms and
  // page table (4-row requests of 64 bf16 heads would otherwise ask for
  // 167 KB); else keys are stored as they are made
  const size_t base = query_lds_bytes<DT, D>(p.rcap, p.Hpad) + (size_t)p.rcap * kHistBins * 4 +
                      (size_t)kFusedMaxPages * 4;
  const size_t kbuf_bytes = (size_t)p.rcap * max_ch * kFusedChunk * 4;
  p.kbuf_stride = mode != 0 && p.rcap * max_ch * kFusedChunk <= kFusedKeyBuf &&
                          base + kbuf_bytes + kFusedStaticLds <= kLdsPerWorkgroup
                      ? max_ch * kFusedChunk
                      : 0;
  const size_t lds = std::max(base + (size_t)p.rcap * p.kbuf_stride * 4, (size_t)kHistBins * 4);
  if (lds + kFusedStaticLds > kLdsPerWorkgroup) return hipErrorInvalidValue;
  if (mode == 0) return launch_fused_as<DT, D, 0>(p, batch, lds, s);
  if (mode == 1) return launch_fused_as<DT, D, 1>(p, batch, lds, s);
  return launch_fused_as<DT, D, 2>(p, batch, lds, s);
}

}  // namespace

bool dsa_indexer_fused_fits(int max_q_per_req, int max_ctx_len) {
  return max_q_per_req <= kFusedMaxRows && max_ctx_len <= kFusedMaxRow;
}

hipError_t dsa_launch_indexer_topk(const DsaIndexerLaunch& a, hipStream_t s) {
  if (a.force_two_pass || !dsa_indexer_fused_fits(a.max_q_per_req, a.max_ctx_len))
    return dsa_launch_indexer_two_pass(a, s);
  FusedParams p;
  p.q_offsets = a.q_offsets;
  p.ctx_lens = a.ctx_lens;
  p.bt = a.block_table;
  p.batch = a.batch;
  p.bt_stride = a.bt_stride;
  p.H = a.n_heads;
  p.Hpad = a.dtype == 0 ? a.n_heads : ((a.n_heads + 15) / 16) * 16;
  p.rcap = a.max_q_per_req;
  p.q = a.q;
  p.q_scale = a.q_scale;
  p.w = a.weights;
  p.k = a.k_cache;
  p.k_scale = a.k_scale;
  p.K = a.topk;
  p.out = a.out_idx;
  p.G = p.row_cap = 0;
  p.keys = reinterpret_cast<uint32_t*>(a.scores);
  p.key_stride = a.score_stride;
  p.counters = a.counters;
  p.hist = a.hist;
  const bool d64 = a.head_dim == 64;
  switch (a.dtype) {
    case 0: return d64 ? launch_fused<0, 64>(p, a.batch, a.max_ctx_len, s) : launch_fused<0, 128>(p, a.batch, a.max_ctx_len, s);
    case 1: return d64 ? launch_fused<1, 64>(p, a.batch, a.max_ctx_len, s) : launch_fused<1, 128>(p, a.batch, a.max_ctx_len, s);
    case 2: return d64 ? launch_fused<2, 64>(p, a.batch, a.max_ctx_len, s) : launch_fused<2, 128>(p, a.batch, a.max_ctx_len, s);
    default: return launch_fused<3, 128>(p, a.batch, a.max_ctx_len, s);  // MXFP8: 128-dim only
  }
}
