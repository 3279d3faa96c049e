// indexer_prefill.hip -- lightning-indexer scores for requests with many
// query rows (chunked prefill, gfx950).
//
// Scoring every visible position for every query row ("Optimizing Inference
// for Hybrid Attention Architectures: From Operator Fusion to Sequence
// Sharding", section "Breaking Down the Computational Path of Hybrid
// Attention", item 1; the prefill route of "Day0 Inference Support and
// Performance Optimization for New LLM Architectures", section III, 3.1) is a
// dense contraction: logits[(row, head)][t] = q[row][head] . k[t] over the
// head dim, i.e. a GEMM of [rows x heads, D] by [D, positions], followed by
// ReLU, the head weights and a sum over heads.
//
// A workgroup owns 4 query rows of one request, one per wave.  A wave keeps
// its row's whole query (64 heads x D) in registers as the MFMA A operand and
// walks the request's positions in tiles of 128, which the four waves share
// through LDS (the next tile's keys are in flight in registers while the
// current one is used).  Per 64 positions a wave runs heads x positions x D
// as 16x16x32 MFMAs into 4 x 4 accumulator tiles, then folds ReLU, the
// weights and the 64-head sum into the accumulators (the heads of a position
// sit in one lane column, so the sum is in-lane plus two lane swaps) and
// writes 64 fp32 scores.  Tiles past the causal edge of the rows are skipped.
// Each row's level-1 digit histogram (top 11 key bits) is complete inside
// the workgroup, so it is stored without atomics for the selection kernel.
#include <algorithm>

#include "dsa_device.h"
#include "indexer_common.h"
#include "radix_select.h"

namespace dsa {

struct PrefillParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* bt;
  int batch, bt_stride;
  int H;
  const void* q;
  const float* q_scale;
  const float* w;
  const void* k;
  const float* k_scale;
  float* scores;
  int64_t score_stride;
  uint32_t* hist;  // [rows][kHistStride]: level-1 histogram at offset 0 (null: scores only)
};

constexpr int kPfThreads = 256;
constexpr int kPfRows = kPfThreads / 64;  // query rows per workgroup
constexpr int kPfTile = 128;              // positions per LDS tile
constexpr int kPfHeads = 64;              // heads held in registers (H is padded to this)

template <int DT, int D>
__global__ __launch_bounds__(kPfThreads, 2) void li_prefill(PrefillParams p) {
  using Gm = IdxGeom<DT, D>;
  using frag_t = typename Gm::frag_t;
  constexpr int ES = Gm::ES;
  constexpr int KS = D / 32;                     // contraction steps
  constexpr int KROW = D * ES + 16;              // padded LDS bytes per key row
  constexpr int TILE_BYTES = kPfTile * D * ES;   // key bytes per tile
  constexpr int VPT = TILE_BYTES / 16 / kPfThreads;  // 16-byte loads per thread per tile
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* ktile = smem;                                              // [kPfTile][KROW]
  float* ksc = reinterpret_cast<float*>(smem + kPfTile * KROW);             // [kPfTile] fp8 scales
  uint32_t* lhist = reinterpret_cast<uint32_t*>(ksc + kPfTile);             // [kPfRows][kHistBins]

  const int b = blockIdx.y;
  const int q0 = p.q_offsets[b], nb = p.q_offsets[b + 1] - q0;
  const int r0 = blockIdx.x * kPfRows;
  if (r0 >= nb) return;
  const int nrows = min(kPfRows, nb - r0);
  const int first_pos = p.ctx_lens[b] - nb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const bool row_ok = wave < nrows;
  const int row = q0 + r0 + wave;                 // this wave's query row
  const int vis_last = first_pos + r0 + nrows;    // positions any row here sees
  const int myvis = row_ok ? first_pos + r0 + wave + 1 : 0;

  for (int c = tid; c < kPfRows * kHistBins; c += kPfThreads) lhist[c] = 0u;

  // this wave's query row as A fragments: qf[mt][ks] = q[row][mt*16 + l16][ks*32 + g*8 ..]
  frag_t qf[kPfHeads / 16][KS];
  float wl[kPfHeads / 16][4];  // weights of heads mt*16 + 4g + i (times the q scale for fp8)
  {
    const unsigned char* qg = static_cast<const unsigned char*>(p.q);
#pragma unroll
    for (int mt = 0; mt < kPfHeads / 16; ++mt) {
      const int h = mt * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        frag_t v{};
        if (row_ok && h < p.H)
          v = *reinterpret_cast<const frag_t*>(qg + ((int64_t)row * p.H + h) * (D * ES) + (ks * 32 + g * 8) * ES);
        qf[mt][ks] = v;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = mt * 16 + 4 * g + i;
        float wv = 0.f;
        if (row_ok && hh < p.H) {
          wv = p.w[(int64_t)row * p.H + hh];
          if (DT == 2) wv *= p.q_scale[(int64_t)row * p.H + hh];
        }
        wl[mt][i] = wv;
      }
    }
  }

  const int ntiles = (vis_last + kPfTile - 1) / kPfTile;
  const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
  const unsigned char* kg = static_cast<const unsigned char*>(p.k);
  uint4 pre[VPT];
  float pre_s = 0.f;
  auto fetch = [&](int tile) {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int c = tid + j * kPfThreads;        // 16-byte piece of the tile
      const int pos = c / (D * ES / 16);         // position within the tile
      const int part = c - pos * (D * ES / 16);
      const int t = tile * kPfTile + pos;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t < vis_last) {  // the block table only covers the request's pages
        const int phys = btrow[t >> 6];
        v = *reinterpret_cast<const uint4*>(kg + ((int64_t)phys * kPage + (t & 63)) * (D * ES) + part * 16);
      }
      pre[j] = v;
    }
    if (DT == 2 && tid < kPfTile) {
      const int t = tile * kPfTile + tid;
      pre_s = t < vis_last ? p.k_scale[(int64_t)btrow[t >> 6] * kPage + (t & 63)] : 0.f;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int c = tid + j * kPfThreads;
      const int pos = c / (D * ES / 16);
      const int part = c - pos * (D * ES / 16);
      *reinterpret_cast<uint4*>(ktile + pos * KROW + part * 16) = pre[j];
    }
    if (DT == 2 && tid < kPfTile) ksc[tid] = pre_s;
  };

  if (ntiles > 0) fetch(0);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();  // the previous tile is no longer read
    stage();
    __syncthreads();
    if (tile + 1 < ntiles) fetch(tile + 1);
    if (!row_ok) continue;
#pragma unroll 1
    for (int sub = 0; sub < kPfTile / 64; ++sub) {
      const int t0 = tile * kPfTile + sub * 64;
      if (t0 >= myvis) break;
      f32x4 acc[kPfHeads / 16][4];
#pragma unroll
      for (int mt = 0; mt < kPfHeads / 16; ++mt)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[mt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        frag_t bf[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          bf[pt] = *reinterpret_cast<const frag_t*>(ktile + (sub * 64 + pt * 16 + l16) * KROW + (ks * 32 + g * 8) * ES);
#pragma unroll
        for (int mt = 0; mt < kPfHeads / 16; ++mt)
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) acc[mt][pt] = mfma_16x16x32(qf[mt][ks], bf[pt], acc[mt][pt]);
      }
      // acc[mt][pt][i] = logit of head mt*16 + 4g + i at position t0 + pt*16 + l16.
      // In-lane head sums per position tile, then a reduce-scatter over the
      // four lane groups that leaves lane (g, l16) with the score of position
      // t0 + 16g + l16; the additions pair the groups as (g0+g1)+(g2+g3), the
      // order the other indexer kernels use, so all routes agree bit for bit.
      float sp[4];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        float s = 0.f;
#pragma unroll
        for (int mt = 0; mt < kPfHeads / 16; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) s += wl[mt][i] * relu_keep_nan(acc[mt][pt][i]);
        sp[pt] = s;
      }
      const bool lo = g & 1, hi = g >> 1;
      // groups g, g^1: lo = 0 keeps tiles 0 and 2, lo = 1 keeps tiles 1 and 3
      const float ka = lo ? sp[1] : sp[0], kb = lo ? sp[3] : sp[2];
      const float sa = lo ? sp[0] : sp[1], sb = lo ? sp[2] : sp[3];
      const float pa = ka + __shfl_xor(sa, 16), pb = kb + __shfl_xor(sb, 16);
      // groups g, g^2: hi = 0 keeps tile lo, hi = 1 keeps tile 2 + lo
      const float keep = hi ? pb : pa, send = hi ? pa : pb;
      float s = keep + __shfl_xor(send, 32);
      const int slot = sub * 64 + g * 16 + l16;
      const int pos = tile * kPfTile + slot;
      if (DT == 2) s *= ksc[slot];
      if (pos < myvis) {
        p.scores[(int64_t)row * p.score_stride + pos] = s;
        atomicAdd(&lhist[wave * kHistBins + (score_key(s) >> kLevelShift[0])], 1u);
      }
    }
  }
  __syncthreads();
  if (!p.hist) return;
  for (int c = tid; c < nrows * kHistBins; c += kPfThreads) {
    const int r = c / kHistBins;
    p.hist[(int64_t)(q0 + r0 + r) * kHistStride + (c - r * kHistBins)] = lhist[c];
  }
}

}  // namespace dsa

using namespace dsa;

template <int DT, int D>
static hipError_t launch_prefill(const PrefillParams& p, dim3 grid, hipStream_t s) {
  using Gm = IdxGeom<DT, D>;
  const size_t lds = (size_t)kPfTile * (D * Gm::ES + 16) + kPfTile * 4 + (size_t)kPfRows * kHistBins * 4;
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(li_prefill<DT, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((li_prefill<DT, D>), grid, dim3(kPfThreads), lds, s, p);
  return hipGetLastError();
}

// The row-tiled kernel runs whole rows per workgroup, so it pays off once the
// rows alone give about one workgroup per compute unit; fewer, longer rows are
// better split by position (li_score).  fp32 keys always go by position.
bool dsa_indexer_rows_route(const DsaIndexerLaunch& a) {
  if (a.dtype == 0 || a.n_heads > kPfHeads) return false;
  if (a.score_route != 0) return a.score_route == 1;
  return a.max_q_per_req > kPfRows && a.num_rows >= 256 * kPfRows;
}

// Scores and level-1 histograms of every row (bf16 or fp8 keys, at most 64
// heads; hipErrorInvalidValue otherwise).
hipError_t dsa_launch_indexer_prefill_scores(const DsaIndexerLaunch& a, hipStream_t s) {
  if (a.dtype == 0 || a.n_heads > kPfHeads) return hipErrorInvalidValue;
  PrefillParams p;
  p.q_offsets = a.q_offsets;
  p.ctx_lens = a.ctx_lens;
  p.bt = a.block_table;
  p.batch = a.batch;
  p.bt_stride = a.bt_stride;
  p.H = a.n_heads;
  p.q = a.q;
  p.q_scale = a.q_scale;
  p.w = a.weights;
  p.k = a.k_cache;
  p.k_scale = a.k_scale;
  p.scores = a.scores;
  p.score_stride = a.score_stride;
  p.hist = a.hist;
  const dim3 grid((a.max_q_per_req + kPfRows - 1) / kPfRows, a.batch);
  const bool d64 = a.head_dim == 64;
  if (a.dtype == 1) return d64 ? launch_prefill<1, 64>(p, grid, s) : launch_prefill<1, 128>(p, grid, s);
  return d64 ? launch_prefill<2, 64>(p, grid, s) : launch_prefill<2, 128>(p, grid, s);
}
