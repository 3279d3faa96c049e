// indexer.hip -- lightning indexer scoring and Top-K selection (gfx950).
//
// Scoring follows "Optimizing Inference for Hybrid Attention Architectures:
// From Operator Fusion to Sequence Sharding", section "Breaking Down the
// Computational Path of Hybrid Attention", item 1: every visible position t
// is scored per indexer head against the query and the heads are combined by
// importance weight,
//     s_t = sum_h w_h * max(q_h . k_t, 0)
// reading keys straight from the paged K cache ("Day0 Inference Support and
// Performance Optimization for New LLM Architectures", section III, 3.1).
//
// Work split.  One workgroup = 4 waves = 4 cache pages (256 positions) of one
// request and up to 4 of its query rows, so the query rows of a request share
// one read of its keys.  bf16 and fp8 keys go through MFMA (heads x positions
// tiles of 16 x 16, contraction over the head dim); fp32 keys use VALU.  Each
// workgroup also histograms the top 11 bits of its scores' order-preserving
// keys per row (LDS, then one global atomic per non-empty bin), which gives
// the selection kernel the first radix level for free.
//
// Selection (li_topk): one 1024-thread workgroup per query row.  From the
// histogram it finds the bin holding the K-th largest key, gathers that bin's
// keys into LDS, resolves the exact K-th key with two more radix levels, then
// makes one ordered pass over the row, keeping every larger key and the
// lowest-position keys equal to the K-th (the tie rule), and writes the kept
// positions in ascending order.
#include <algorithm>
#include <type_traits>

#include "dsa_device.h"

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
  uint32_t* hist;
};

constexpr int kRowsPerBlock = 4;
constexpr int kScoreThreads = 256;  // 4 waves, one page each
constexpr int kChunk = 256;         // positions per workgroup

// ReLU that lets NaN through (NaN < 0 is false), so a stray read of poisoned
// cache data shows up in the result instead of vanishing.
__device__ __forceinline__ float relu_keep_nan(float v) { return v < 0.f ? 0.f : v; }

__device__ __forceinline__ f32x4 mfma_16x16x32(uint4 a, uint4 b, f32x4 c, bf16x8*) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_16x16x32(uint2 a, uint2 b, f32x4 c, uint8_t*) {
  long la = __builtin_bit_cast(long, a), lb = __builtin_bit_cast(long, b);
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(la, lb, c, 0, 0, 0);
}

// Common prologue: decode the block's request, rows and causal bounds.
struct BlockRows {
  int b, q0, nb, r0, nrows, first_pos, pos_max, c0;
};

__device__ __forceinline__ bool block_rows(const LiParams& p, BlockRows& br) {
  br.b = blockIdx.z;
  br.q0 = p.q_offsets[br.b];
  br.nb = p.q_offsets[br.b + 1] - br.q0;
  br.r0 = blockIdx.y * kRowsPerBlock;
  if (br.r0 >= br.nb) return false;
  br.nrows = min(kRowsPerBlock, br.nb - br.r0);
  br.first_pos = p.ctx_lens[br.b] - br.nb;          // position of the request's first query row
  br.pos_max = br.first_pos + br.r0 + br.nrows - 1;  // last position any row here may see
  br.c0 = blockIdx.x * kChunk;
  return br.c0 <= br.pos_max;
}

// Write one score and count it in the row's LDS histogram.
__device__ __forceinline__ void emit_score(const LiParams& p, const BlockRows& br, uint32_t* hl,
                                           int r, int pos, float s) {
  if (pos <= br.first_pos + br.r0 + r) {
    p.scores[(int64_t)(br.q0 + br.r0 + r) * p.score_stride + pos] = s;
    atomicAdd(&hl[r * kHistBins + (score_key(s) >> (32 - kHistBits))], 1u);
  }
}

__device__ __forceinline__ void flush_hist(const LiParams& p, const BlockRows& br, const uint32_t* hl) {
  for (int c = threadIdx.x; c < br.nrows * kHistBins; c += kScoreThreads) {
    uint32_t v = hl[c];
    if (v) {
      int r = c / kHistBins, bin = c - r * kHistBins;
      atomicAdd(&p.hist[(int64_t)(br.q0 + br.r0 + r) * kHistBins + bin], v);
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA scoring for bf16 (DT = 1) and fp8 e4m3 (DT = 2) keys, head dim D.
// Logit tile: D[m = head][n = position] = sum_k Q[head][k] * K[position][k],
// A = query rows from LDS, B = keys straight from the page in HBM (each lane
// loads 8 consecutive elements of one key row).
// ---------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(kScoreThreads) void li_score_mfma(LiParams p) {
  constexpr int ES = (DT == 1) ? 2 : 1;        // bytes per element
  constexpr int QSTRIDE = D * ES + 16;         // LDS bytes per (row, head), padded
  constexpr int KS = D / 32;                   // contraction steps
  using frag_t = typename std::conditional<DT == 1, uint4, uint2>::type;
  using tag_t = typename std::conditional<DT == 1, bf16x8, uint8_t>::type;

  BlockRows br;
  if (!block_rows(p, br)) return;
  extern __shared__ __align__(16) unsigned char smem[];
  const int Hpad = p.Hpad;
  unsigned char* qs = smem;
  float* wsm = reinterpret_cast<float*>(smem + p.rcap * Hpad * QSTRIDE);
  uint32_t* hl = reinterpret_cast<uint32_t*>(wsm + p.rcap * Hpad);
  const int tid = threadIdx.x;

  {  // stage the rows' queries (heads past H zero-filled) and folded weights
    constexpr int CPH = D * ES / 16;  // 16-byte chunks per head
    const int total = br.nrows * Hpad * CPH;
    const unsigned char* qg = static_cast<const unsigned char*>(p.q);
    for (int c = tid; c < total; c += kScoreThreads) {
      int r = c / (Hpad * CPH);
      int rem = c - r * Hpad * CPH;
      int h = rem / CPH, part = rem - h * CPH;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (h < p.H)
        v = *reinterpret_cast<const uint4*>(qg + ((int64_t)(br.q0 + br.r0 + r) * p.H + h) * (D * ES) + part * 16);
      *reinterpret_cast<uint4*>(qs + (r * Hpad + h) * QSTRIDE + part * 16) = v;
    }
    for (int c = tid; c < br.nrows * Hpad; c += kScoreThreads) {
      int r = c / Hpad, h = c - r * Hpad;
      float wv = 0.f;
      if (h < p.H) {
        int64_t o = (int64_t)(br.q0 + br.r0 + r) * p.H + h;
        wv = p.w[o];
        if (DT == 2) wv *= p.q_scale[o];  // q scale > 0 folds through the ReLU
      }
      wsm[r * Hpad + h] = wv;
    }
    for (int c = tid; c < br.nrows * kHistBins; c += kScoreThreads) hl[c] = 0u;
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int pg = (br.c0 >> 6) + wave;  // logical page handled by this wave
  const int p0 = pg * kPage;
  if (p0 <= br.pos_max) {
    const int phys = p.bt[(int64_t)br.b * p.bt_stride + pg];
    const unsigned char* kp = static_cast<const unsigned char*>(p.k) + (int64_t)phys * kPage * D * ES;
    frag_t kf[4][KS];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[pt][ks] = *reinterpret_cast<const frag_t*>(kp + ((pt * 16 + l16) * D + ks * 32 + g * 8) * ES);
    float kscale[4];
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
      kscale[pt] = (DT == 2) ? p.k_scale[(int64_t)phys * kPage + pt * 16 + l16] : 1.f;

    for (int r = 0; r < br.nrows; ++r) {
      float sacc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int ht = 0; ht < Hpad / 16; ++ht) {
        f32x4 acc[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const unsigned char* qrow = qs + (r * Hpad + ht * 16 + l16) * QSTRIDE + g * 8 * ES;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          frag_t a = *reinterpret_cast<const frag_t*>(qrow + ks * 32 * ES);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) acc[pt] = mfma_16x16x32(a, kf[pt][ks], acc[pt], (tag_t*)nullptr);
        }
        // acc[pt][i] = logit of head ht*16 + 4g + i at position pt*16 + l16
        const float* wr = wsm + r * Hpad + ht * 16 + 4 * g;
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sacc[pt] += wr[i] * relu_keep_nan(acc[pt][i]);
      }
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        float s = sacc[pt];
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        s *= kscale[pt];
        if (g == 0) emit_score(p, br, hl, r, p0 + pt * 16 + l16, s);
      }
    }
  }
  __syncthreads();
  flush_hist(p, br, hl);
}

// ---------------------------------------------------------------------------
// fp32 scoring on VALU: one thread per position, its key row in registers,
// queries and weights broadcast from LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kScoreThreads) void li_score_f32(LiParams p) {
  BlockRows br;
  if (!block_rows(p, br)) return;
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = p.H;
  float* qs = reinterpret_cast<float*>(smem);                // [rows][H][D]
  float* wsm = qs + p.rcap * H * D;                          // [rows][H]
  uint32_t* hl = reinterpret_cast<uint32_t*>(wsm + p.rcap * H);
  const int tid = threadIdx.x;
  const float* qg = static_cast<const float*>(p.q);
  for (int c = tid; c < br.nrows * H * D; c += kScoreThreads)
    qs[c] = qg[(int64_t)(br.q0 + br.r0) * H * D + c];
  for (int c = tid; c < br.nrows * H; c += kScoreThreads)
    wsm[c] = p.w[(int64_t)(br.q0 + br.r0) * H + c];
  for (int c = tid; c < br.nrows * kHistBins; c += kScoreThreads) hl[c] = 0u;
  __syncthreads();

  const int pos = br.c0 + tid;
  if (pos <= br.pos_max) {
    const int phys = p.bt[(int64_t)br.b * p.bt_stride + (pos >> 6)];
    const float4* krow = reinterpret_cast<const float4*>(static_cast<const float*>(p.k) +
                                                         ((int64_t)phys * kPage + (pos & 63)) * D);
    float4 kr[D / 4];
#pragma unroll
    for (int d = 0; d < D / 4; ++d) kr[d] = krow[d];
    for (int r = 0; r < br.nrows; ++r) {
      float s = 0.f;
      for (int h = 0; h < H; ++h) {
        const float4* qh = reinterpret_cast<const float4*>(qs + (r * H + h) * D);
        float logit = 0.f;
#pragma unroll
        for (int d = 0; d < D / 4; ++d) {
          float4 qv = qh[d];
          logit = fmaf(qv.x, kr[d].x, logit);
          logit = fmaf(qv.y, kr[d].y, logit);
          logit = fmaf(qv.z, kr[d].z, logit);
          logit = fmaf(qv.w, kr[d].w, logit);
        }
        s = fmaf(wsm[r * H + h], relu_keep_nan(logit), s);
      }
      emit_score(p, br, hl, r, pos, s);
    }
  }
  __syncthreads();
  flush_hist(p, br, hl);
}

__global__ void fill_u32(uint32_t* x, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    x[i] = v;
}

// ---------------------------------------------------------------------------
// Selection
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kCandCap = 12288;
constexpr int kItems = 4;  // consecutive positions per thread per pass

struct TopkParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  int batch;
  const float* scores;
  int64_t score_stride;
  const uint32_t* hist;
  int K;
  int32_t* out;
};

struct TopkShared {
  uint32_t bins[kHistBins];
  uint32_t cand[kCandCap];
  int wave_sum[kTopkWaves];
  int ncand;
  int res_bin, res_above;
};

// Largest bin index `bin` such that the keys in bins >= bin number at least k;
// `above` = keys in bins > bin.  Wave 0 scans from the top; result in sh.
__device__ void kth_bin(TopkShared& sh, int nbins, int k) {
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    if (lane == 0) {  // defaults if the counts fall short of k (inconsistent input)
      sh.res_bin = 0;
      sh.res_above = 0;
    }
    const int per = nbins / 64;
    const int hi = nbins - lane * per;  // this lane owns bins [hi - per, hi)
    int local = 0;
    for (int x = hi - per; x < hi; ++x) local += sh.bins[x];
    int incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    const int before = incl - local;
    if (before < k && incl >= k) {
      int acc = before;
      for (int x = hi - 1; x >= hi - per; --x) {
        int c = sh.bins[x];
        if (acc + c >= k) {
          sh.res_bin = x;
          sh.res_above = acc;
          break;
        }
        acc += c;
      }
    }
  }
  __syncthreads();
}

// Exclusive prefix of v over the workgroup (position order = thread order);
// returns the prefix, writes the total.
__device__ __forceinline__ int block_excl_scan(TopkShared& sh, int v, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int t = __shfl_up(incl, off);
    if (lane >= off) incl += t;
  }
  __syncthreads();
  if (lane == 63) sh.wave_sum[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w2 = 0; w2 < kTopkWaves; ++w2) {
    int s = sh.wave_sum[w2];
    if (w2 < wave) base += s;
    total += s;
  }
  return base + incl - v;
}

__device__ __forceinline__ void load_keys(const float* row, int t0, int vis, uint32_t key[kItems],
                                          bool valid[kItems]) {
  if (t0 + kItems <= vis) {
    float4 v = *reinterpret_cast<const float4*>(row + t0);
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

__global__ __launch_bounds__(kTopkThreads) void li_topk(TopkParams p) {
  __shared__ TopkShared sh;
  const int i = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63;
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int nb = p.q_offsets[b + 1] - p.q_offsets[b];
  const int vis = p.ctx_lens[b] - nb + (i - p.q_offsets[b]) + 1;
  const int K = p.K;
  int32_t* out = p.out + (int64_t)i * K;
  if (vis <= K) {  // everything visible is kept
    for (int t = tid; t < K; t += kTopkThreads) out[t] = t < vis ? t : -1;
    return;
  }
  const float* row = p.scores + (int64_t)i * p.score_stride;

  // level 1: the histogram the scoring kernel built (top 11 key bits)
  for (int c = tid; c < kHistBins; c += kTopkThreads) sh.bins[c] = p.hist[(int64_t)i * kHistBins + c];
  if (tid == 0) sh.ncand = 0;
  __syncthreads();
  kth_bin(sh, kHistBins, K);
  const uint32_t bin1 = sh.res_bin;
  int need = K - sh.res_above;          // keys still needed from bin1 (>= 1)
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
        bool pred = valid[e] && (key[e] >> 21) == bin1;
        uint64_t m = __ballot(pred);
        int n = __popcll(m);
        int base = 0;
        if (n) {
          if (lane == 0) base = atomicAdd(&sh.ncand, n);
          base = __shfl(base, 0);
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
  for (int level = 0; level < 2; ++level) {
    const int nbins = level == 0 ? 2048 : 1024;
    const int shift = level == 0 ? 10 : 0;
    for (int c = tid; c < nbins; c += kTopkThreads) sh.bins[c] = 0u;
    __syncthreads();
    if (in_lds) {
      for (int c = tid; c < ncand; c += kTopkThreads) {
        uint32_t low = sh.cand[c];
        if (level == 0 || (low >> 10) == (prefix & 2047u)) atomicAdd(&sh.bins[(low >> shift) & (nbins - 1)], 1u);
      }
    } else {
      for (int t0 = tid * kItems; t0 < vis; t0 += kTopkThreads * kItems) {
        uint32_t key[kItems];
        bool valid[kItems];
        load_keys(row, t0, vis, key, valid);
#pragma unroll
        for (int e = 0; e < kItems; ++e) {
          bool hit = valid[e] && (level == 0 ? (key[e] >> 21) == bin1 : (key[e] >> 10) == prefix);
          if (hit) atomicAdd(&sh.bins[(key[e] >> shift) & (nbins - 1)], 1u);
        }
      }
    }
    __syncthreads();
    kth_bin(sh, nbins, need);
    prefix = (prefix << (level == 0 ? 11 : 10)) | (uint32_t)sh.res_bin;
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
    if (t0 < vis) load_keys(row, t0, vis, key, valid);
    else {
#pragma unroll
      for (int e = 0; e < kItems; ++e) { valid[e] = false; key[e] = 0u; }
    }
    int neq = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) neq += (valid[e] && key[e] == kth);
    int eq_total;
    int eq_before = block_excl_scan(sh, neq, eq_total) + eq_run;
    bool sel[kItems];
    int nsel = 0;
#pragma unroll
    for (int e = 0; e < kItems; ++e) {
      bool is_eq = valid[e] && key[e] == kth;
      sel[e] = (valid[e] && key[e] > kth) || (is_eq && eq_before < need);
      eq_before += is_eq;
      nsel += sel[e];
    }
    int sel_total;
    int pos = block_excl_scan(sh, nsel, sel_total) + written;
#pragma unroll
    for (int e = 0; e < kItems; ++e)
      if (sel[e] && pos < K) out[pos++] = t0 + e;
    eq_run += eq_total;
    written += sel_total;
  }
  for (int t = written + tid; t < K; t += kTopkThreads) out[t] = -1;  // unreachable when vis > K
}

}  // namespace dsa

using namespace dsa;

static size_t score_lds_bytes(int dtype, int rcap, int Hpad, int D) {
  const size_t per_head = dtype == 0 ? (size_t)D * 4 : (size_t)D * (dtype == 1 ? 2 : 1) + 16;
  return (size_t)rcap * (Hpad * per_head + Hpad * 4 + kHistBins * 4);
}

template <typename K>
static hipError_t launch_dyn(K kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s, const LiParams& p) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kernel, grid, block, lds, s, p);
  return hipGetLastError();
}

hipError_t dsa_launch_indexer_topk(const DsaIndexerLaunch& a, hipStream_t s) {
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

  const int64_t nhist = (int64_t)a.num_rows * kHistBins;
  hipLaunchKernelGGL(fill_u32, dim3((unsigned)std::min<int64_t>((nhist + 255) / 256, 4096)), dim3(256), 0, s,
                     a.hist, nhist, 0u);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  dim3 grid((a.max_ctx_len + kChunk - 1) / kChunk, (a.max_q_per_req + kRowsPerBlock - 1) / kRowsPerBlock,
            a.batch);
  const size_t lds = score_lds_bytes(a.dtype, p.rcap, p.Hpad, a.head_dim);
  if (a.dtype == 0) {
    e = a.head_dim == 64 ? launch_dyn(li_score_f32<64>, grid, dim3(kScoreThreads), lds, s, p)
                         : launch_dyn(li_score_f32<128>, grid, dim3(kScoreThreads), lds, s, p);
  } else if (a.dtype == 1) {
    e = a.head_dim == 64 ? launch_dyn(li_score_mfma<1, 64>, grid, dim3(kScoreThreads), lds, s, p)
                         : launch_dyn(li_score_mfma<1, 128>, grid, dim3(kScoreThreads), lds, s, p);
  } else {
    e = a.head_dim == 64 ? launch_dyn(li_score_mfma<2, 64>, grid, dim3(kScoreThreads), lds, s, p)
                         : launch_dyn(li_score_mfma<2, 128>, grid, dim3(kScoreThreads), lds, s, p);
  }
  if (e != hipSuccess) return e;

  TopkParams tp;
  tp.q_offsets = a.q_offsets;
  tp.ctx_lens = a.ctx_lens;
  tp.batch = a.batch;
  tp.scores = a.scores;
  tp.score_stride = a.score_stride;
  tp.hist = a.hist;
  tp.K = a.topk;
  tp.out = a.out_idx;
  hipLaunchKernelGGL(li_topk, dim3(a.num_rows), dim3(kTopkThreads), 0, s, tp);
  return hipGetLastError();
}
