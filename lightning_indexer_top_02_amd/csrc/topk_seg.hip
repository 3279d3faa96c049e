// topk_seg.hip -- Top-K selection of the two-pass indexer route, parallel
// over segments of each score row (gfx950).
//
// Selection keeps, per query row, the K highest scores among its visible
// positions, ties to the lower position, written in ascending position order
// ("Optimizing Inference for Hybrid Attention Architectures: From Operator
// Fusion to Sequence Sharding", section "Breaking Down the Computational
// Path of Hybrid Attention", item 1; the order is the "index rearrangement"
// of "Optimizing Inference for Hybrid Attention LLMs: Practices for Fast
// Adaptation", section 3, item 2).
//
// The scoring kernel has already left each row's histogram of the top 11
// key bits in the workspace.  A row is then cut into segments of 8192
// positions and handled by three kernels:
//   li_seg_gather  (a workgroup per segment): finds the histogram bin that
//                  holds the K-th key, counts the segment's keys above it,
//                  marks them in a bitmap of the row's kept positions and
//                  appends the keys of that bin (low 21 bits and position)
//                  to the row's candidate list;
//   li_seg_resolve (a workgroup per row): two more radix digits over the
//                  candidates give the K-th key exactly; if fewer keys equal
//                  to it are kept than exist, a radix select over their
//                  positions gives the last kept position; the kept
//                  candidates are marked in the bitmap and per-segment kept
//                  counts become output offsets;
//   li_seg_write   (a workgroup per segment): writes the kept positions of
//                  its segment at its offset, in order, from the bitmap, so
//                  the scores are read only once.
// Thread t of a segment reads positions s0 + R c + 4 t + e (c < 8, e < 4,
// R = 4 x the segment's threads): each wave load is 1 KB of consecutive
// scores, with no staging buffer.  Bit 4 c + e of the segment's bitmap word t
// marks that position; li_seg_write regathers the bits of 32 consecutive
// positions per thread.
// A row whose boundary bin holds more keys than the candidate list can take
// (heavy ties) is flagged and selected whole by li_seg_resolve's workgroup
// (select_whole_row), and li_seg_write leaves it alone.  The per-row state
// lives in the unused tail of the row's histogram block; the histogram and
// the candidate counter are zero again when the three kernels are done.
#include <algorithm>

#include "dsa_device.h"
#include "radix_select.h"

namespace dsa {

constexpr int kSegLen = 8192;                     // positions per segment
constexpr int kSegThreads = kSegLen / 32;         // one bitmap word of 32 positions per thread
constexpr int kSegRound = 4 * kSegThreads;        // positions of one 16-byte load per thread
constexpr int kResolveThreads = 1024;
// words of a row's histogram block (kHistStride) after the level-1 bins
constexpr int kSegBase = kHistBins;               // per-segment counts, then offsets
constexpr int kStateCount = kHistStride - 4;      // candidates appended (zero between calls)
constexpr int kStateKth = kHistStride - 3;        // the K-th key
constexpr int kStateLimit = kHistStride - 2;      // last kept position among keys equal to it
constexpr int kStateFlags = kHistStride - 1;      // 1: row left to the one-workgroup path
constexpr int kMaxSegs = kStateCount - kSegBase;  // longest row: kMaxSegs * kSegLen positions

struct SegParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  int batch;
  const float* scores;
  int64_t score_stride;
  uint32_t* hist;
  int K;
  int32_t* out;
  uint32_t* cand_key;  // [rows][cand_cap] low 21 key bits
  int32_t* cand_pos;   // [rows][cand_cap] positions
  int cand_cap;
  uint32_t* keep;      // [rows][keep_words] bitmap of the kept positions (layout above)
};

// Bitmap words per row: kSegLen / 32 per segment of the score stride.
__host__ __device__ constexpr int64_t keep_words(int64_t score_stride) {
  return (score_stride + kSegLen - 1) / kSegLen * (kSegLen / 32);
}

// Word and bit of position pos in its row's bitmap.
__device__ __forceinline__ void keep_bit(int pos, int& word, int& bit) {
  const int seg = pos / kSegLen, o = pos - seg * kSegLen;
  word = seg * (kSegLen / 32) + ((o % kSegRound) >> 2);
  bit = 4 * (o / kSegRound) + (o & 3);
}

__device__ __forceinline__ int visible_of(const SegParams& p, int i) {
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int nb = p.q_offsets[b + 1] - p.q_offsets[b];
  return p.ctx_lens[b] - nb + (i - p.q_offsets[b]) + 1;
}

// Sum over the workgroup (result valid in every thread).
template <int NT>
__device__ __forceinline__ int block_sum(int v, int* wsum) {
  int total;
  block_excl_scan<NT>(v, total, wsum);
  return total;
}

static_assert(kSegThreads * 32 == kSegLen && kSegThreads % 64 == 0, "whole waves, a bitmap word per thread");

__global__ __launch_bounds__(kSegThreads) void li_seg_gather(SegParams p) {
  __shared__ __align__(16) int wsum[kSegThreads / 64];
  __shared__ int sh[3];
  const int i = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const int vis = visible_of(p, i);
  const int s0 = seg * kSegLen;
  if (vis <= p.K || s0 >= vis) return;
  uint32_t* hrow = p.hist + (int64_t)i * kHistStride;
  // waves 1-3 issue their score loads at once; wave 0 first finds the
  // boundary bin in the row's histogram, then issues its own (its bins and
  // scores are never live together, which keeps the register count low)
  const float* row = p.scores + (int64_t)i * p.score_stride;
  float4 v[8];
  auto load_scores = [&]() {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int t = s0 + kSegRound * c + 4 * tid;
      v[c] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t + 4 <= vis) {
        v[c] = *reinterpret_cast<const float4*>(row + t);
      } else {
        if (t < vis) v[c].x = row[t];
        if (t + 1 < vis) v[c].y = row[t + 1];
        if (t + 2 < vis) v[c].z = row[t + 2];
      }
    }
  };
  if (tid >= 64) {
    load_scores();
  } else {
    int bin, above, total, count;
    kth_bin_wave_count<32>(hrow, p.K, bin, above, total, count);
    if (tid == 0) {
      sh[0] = bin;
      sh[1] = count;
    }
    load_scores();
  }
  __syncthreads();
  const uint32_t bin1 = (uint32_t)sh[0];
  const bool gather = sh[1] <= p.cand_cap;
  // key of element b of this thread (0 past the row; the callers also test t < vis)
  auto key_of = [&](int b) {
    const float4 q = v[b >> 2];
    const float x = (b & 3) == 0 ? q.x : ((b & 3) == 1 ? q.y : ((b & 3) == 2 ? q.z : q.w));
    return score_key(x);
  };
  // bit 4c + e of gtm / eqm: position s0 + kSegRound c + 4 tid + e is visible and
  // lies above / in the boundary bin
  const int lim = vis - s0 - 4 * tid;
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const bool ok = kSegRound * (b >> 2) + (b & 3) < lim;
    const uint32_t d = key_of(b) >> kLevelShift[0];
    gtm |= ok && d > bin1 ? 1u << b : 0u;
    eqm |= ok && d == bin1 ? 1u << b : 0u;
  }
  const int ngt = __popc(gtm), neq = __popc(eqm);
  // li_seg_resolve adds the kept candidates to the bitmap
  if (gather) p.keep[i * keep_words(p.score_stride) + seg * (kSegLen / 32) + tid] = gtm;
  // keys above the boundary bin: a count per segment
  const int gt_total = block_sum<kSegThreads>(ngt, wsum);
  if (tid == 0) hrow[kSegBase + seg] = (uint32_t)gt_total;
  if (!gather) return;
  // keys of the boundary bin: appended to the row's candidate list
  int eq_total;
  const int eq_before = block_excl_scan<kSegThreads>(neq, eq_total, wsum);
  if (tid == 0) sh[2] = eq_total ? (int)atomicAdd(&hrow[kStateCount], (uint32_t)eq_total) : 0;
  __syncthreads();
  int o = sh[2] + eq_before;
  uint32_t* ck = p.cand_key + (int64_t)i * p.cand_cap;
  int32_t* cp = p.cand_pos + (int64_t)i * p.cand_cap;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    if ((eqm >> b) & 1u) {
      if (o < p.cand_cap) {
        ck[o] = key_of(b) & 0x1fffffu;
        cp[o] = s0 + kSegRound * (b >> 2) + 4 * tid + (b & 3);
      }
      ++o;
    }
  }
}

// ---------------------------------------------------------------------------
// One-workgroup selection of a whole row
// ---------------------------------------------------------------------------
constexpr int kTopkThreads = 1024;
constexpr int kCandCap = 12288;
constexpr int kItems = 4;  // consecutive positions per thread per pass

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

// The whole row in one 1024-thread workgroup (rows whose boundary bin holds
// more keys than the candidate list takes: heavy ties).  It finds the bin
// holding the K-th largest key from the row's histogram, gathers that bin's
// keys into LDS when they fit, resolves the exact K-th key with two more
// radix levels, then makes one ordered pass keeping every larger key and the
// lowest-position keys equal to the K-th (the tie rule), writing positions
// in ascending order.  It zeroes the row's level-1 bins on the way out.
__device__ void select_whole_row(const float* row, int vis, int K, int32_t* out, uint32_t* hrow,
                                 TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;

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

struct ResolveShared {
  uint32_t bins[kHistBins];
  uint32_t segc[kMaxSegs];
  alignas(16) int wsum[kResolveThreads / 64];
  int res[2];
};

// k-th largest bin of the histogram in sh.bins (wave 0), broadcast.
template <int PER>
__device__ __forceinline__ void resolve_kth(ResolveShared& sh, int k, int& bin, int& above) {
  if (threadIdx.x < 64) {
    int b, a, t;
    kth_bin_wave<PER>(sh.bins, k, b, a, t);
    if (threadIdx.x == 0) {
      sh.res[0] = b;
      sh.res[1] = a;
    }
  }
  __syncthreads();
  bin = sh.res[0];
  above = sh.res[1];
  __syncthreads();
}

__global__ __launch_bounds__(kResolveThreads) void li_seg_resolve(SegParams p) {
  static_assert(kResolveThreads == kTopkThreads, "flagged rows are selected by the same workgroup");
  __shared__ union {
    ResolveShared r;
    TopkShared t;
  } shu;
  ResolveShared& sh = shu.r;
  const int i = blockIdx.x, tid = threadIdx.x;
  const int vis = visible_of(p, i);
  uint32_t* hrow = p.hist + (int64_t)i * kHistStride;
  if (vis <= p.K) {  // every visible position is kept (written by li_seg_write)
    for (int c = tid; c < kHistBins; c += kResolveThreads) hrow[c] = 0u;
    return;
  }
  const int K = p.K;
  for (int c = tid; c < kHistBins; c += kResolveThreads) sh.bins[c] = hrow[c];
  __syncthreads();
  int bin1, above;
  resolve_kth<32>(sh, K, bin1, above);
  const int ncand = (int)sh.bins[bin1];
  __syncthreads();  // every thread has read it before the bins are reused
  if (ncand > p.cand_cap) {  // the whole row here, in this workgroup (clears the bins)
    if (tid == 0) hrow[kStateFlags] = 1u;  // (li_seg_write skips the row)
    select_whole_row(p.scores + (int64_t)i * p.score_stride, vis, K, p.out + (int64_t)i * K, hrow, shu.t);
    return;
  }
  int need = K - above;  // keys still needed from bin1 (>= 1)
  const uint32_t* ck = p.cand_key + (int64_t)i * p.cand_cap;
  const int32_t* cp = p.cand_pos + (int64_t)i * p.cand_cap;

  // key bits 20..10, then 9..0, over the candidates
  for (int c = tid; c < kHistBins; c += kResolveThreads) sh.bins[c] = 0u;
  __syncthreads();
  for (int c = tid; c < ncand; c += kResolveThreads) atomicAdd(&sh.bins[ck[c] >> 10], 1u);
  __syncthreads();
  int b2, a2;
  resolve_kth<32>(sh, need, b2, a2);
  need -= a2;
  for (int c = tid; c < kHistBins; c += kResolveThreads) sh.bins[c] = 0u;
  __syncthreads();
  for (int c = tid; c < ncand; c += kResolveThreads) {
    const uint32_t k = ck[c];
    if ((k >> 10) == (uint32_t)b2) atomicAdd(&sh.bins[k & 1023u], 1u);
  }
  __syncthreads();
  int b3, a3;
  resolve_kth<16>(sh, need, b3, a3);
  need -= a3;
  const uint32_t low = ((uint32_t)b2 << 10) | (uint32_t)b3;  // low 21 bits of the K-th key
  const int n_eq = (int)sh.bins[b3];
  __syncthreads();

  // the last kept position among the n_eq keys equal to the K-th: the
  // need-th smallest of their positions, i.e. the (n_eq - need + 1)-th
  // largest, found 11, 11 and 9 bits at a time
  int limit = 0x7fffffff;
  if (need < n_eq) {
    int kk = n_eq - need + 1;
    uint32_t pprefix = 0u;
    for (int level = 0; level < 3; ++level) {
      const int shift = level == 0 ? 20 : (level == 1 ? 9 : 0);
      const int pshift = level == 1 ? 20 : 9;  // the previous level's shift
      const uint32_t mask = level == 2 ? 511u : 2047u;
      for (int c = tid; c < kHistBins; c += kResolveThreads) sh.bins[c] = 0u;
      __syncthreads();
      for (int c = tid; c < ncand; c += kResolveThreads) {
        const uint32_t pos = (uint32_t)cp[c];
        const bool match = ck[c] == low && (level == 0 || (pos >> pshift) == pprefix);
        if (match) atomicAdd(&sh.bins[(pos >> shift) & mask], 1u);
      }
      __syncthreads();
      int pb, pa;
      if (level == 2) resolve_kth<8>(sh, kk, pb, pa);
      else resolve_kth<32>(sh, kk, pb, pa);
      kk -= pa;
      pprefix = level == 0 ? (uint32_t)pb : ((pprefix << (level == 1 ? 11 : 9)) | (uint32_t)pb);
    }
    limit = (int)pprefix;
  }

  // kept candidates per segment, plus the keys above bin1: output offsets
  const int nseg = (vis + kSegLen - 1) / kSegLen;
  for (int s = tid; s < nseg; s += kResolveThreads) sh.segc[s] = hrow[kSegBase + s];
  __syncthreads();
  uint32_t* keep = p.keep + i * keep_words(p.score_stride);
  for (int c = tid; c < ncand; c += kResolveThreads) {
    const uint32_t k = ck[c];
    const int pos = cp[c];
    if (k > low || (k == low && pos <= limit)) {
      atomicAdd(&sh.segc[pos / kSegLen], 1u);
      int word, bit;
      keep_bit(pos, word, bit);
      atomicOr(&keep[word], 1u << bit);
    }
  }
  __syncthreads();
  constexpr int kPerT = (kMaxSegs + kResolveThreads - 1) / kResolveThreads;
  int v[kPerT], sum = 0;
#pragma unroll
  for (int j = 0; j < kPerT; ++j) {
    const int s = tid * kPerT + j;
    v[j] = s < nseg ? (int)sh.segc[s] : 0;
    sum += v[j];
  }
  int total;
  int run = block_excl_scan<kResolveThreads>(sum, total, sh.wsum);
#pragma unroll
  for (int j = 0; j < kPerT; ++j) {
    const int s = tid * kPerT + j;
    if (s < nseg) hrow[kSegBase + s] = (uint32_t)run;
    run += v[j];
  }
  if (tid == 0) {
    hrow[kStateKth] = ((uint32_t)bin1 << 21) | low;
    hrow[kStateLimit] = (uint32_t)limit;
    hrow[kStateFlags] = 0u;
    hrow[kStateCount] = 0u;
  }
  for (int c = tid; c < kHistBins; c += kResolveThreads) hrow[c] = 0u;
}

__global__ __launch_bounds__(kSegThreads) void li_seg_write(SegParams p) {
  __shared__ __align__(16) int wsum[kSegThreads / 64];
  const int i = blockIdx.y, seg = blockIdx.x, tid = threadIdx.x;
  const int vis = visible_of(p, i);
  const int K = p.K;
  int32_t* out = p.out + (int64_t)i * K;
  if (vis <= K) {
    for (int t = seg * kSegLen + tid; t < min(K, (seg + 1) * kSegLen); t += kSegThreads) out[t] = t < vis ? t : -1;
    return;
  }
  const uint32_t* hrow = p.hist + (int64_t)i * kHistStride;
  const int s0 = seg * kSegLen;
  if (s0 >= vis) return;
  // the kept positions are the set bits of the row's bitmap (the keys
  // above the boundary bin, from li_seg_gather, and the kept candidates,
  // from li_seg_resolve); thread t takes positions s0 + 32 t .. + 31, whose
  // bits are bits 4c .. 4c + 3 (c = t / (kSegRound / 32)) of the segment's
  // words 8 (t % (kSegRound / 32)) .. + 7
  const int pos0 = s0 + tid * 32;
  uint32_t sel = 0u;
  if (pos0 < vis) {
    const uint4* w4 = reinterpret_cast<const uint4*>(p.keep + i * keep_words(p.score_stride) + seg * (kSegLen / 32) +
                                                     8 * (tid % (kSegRound / 32)));
    const uint4 a = w4[0], b = w4[1];
    const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    const int c4 = 4 * (tid / (kSegRound / 32));
#pragma unroll
    for (int m = 0; m < 8; ++m) sel |= ((w[m] >> c4) & 0xfu) << (4 * m);
  }
  if (hrow[kStateFlags] & 1u) return;  // (uniform) the row was selected whole by li_seg_resolve
  const int off = (int)hrow[kSegBase + seg];
  int total;
  int o = off + block_excl_scan<kSegThreads>(__popc(sel), total, wsum);
  while (sel != 0u) {
    const int c = __builtin_ctz(sel);
    if (o < K) out[o] = pos0 + c;
    ++o;
    sel &= sel - 1u;
  }
}

}  // namespace dsa

using namespace dsa;

int dsa_seg_max_segments() { return kMaxSegs; }
int dsa_seg_length() { return kSegLen; }
int dsa_seg_cand_cap(int max_ctx_len) { return std::min((max_ctx_len + 255) / 256 * 256, 8192); }
int64_t dsa_seg_keep_words(int64_t score_stride) { return keep_words(score_stride); }

// The three segment kernels (flagged rows are selected inside li_seg_resolve).
hipError_t dsa_launch_topk_segments(const DsaIndexerLaunch& a, hipStream_t s) {
  SegParams p;
  p.q_offsets = a.q_offsets;
  p.ctx_lens = a.ctx_lens;
  p.batch = a.batch;
  p.scores = a.scores;
  p.score_stride = a.score_stride;
  p.hist = a.hist;
  p.K = a.topk;
  p.out = a.out_idx;
  p.cand_key = a.cand_key;
  p.cand_pos = a.cand_pos;
  p.cand_cap = a.cand_cap;
  p.keep = a.keep_bits;
  const int nseg = (a.max_ctx_len + kSegLen - 1) / kSegLen;
  const dim3 grid(nseg, a.num_rows);
  hipLaunchKernelGGL(li_seg_gather, grid, dim3(kSegThreads), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(li_seg_resolve, dim3(a.num_rows), dim3(kResolveThreads), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(li_seg_write, grid, dim3(kSegThreads), 0, s, p);
  return hipGetLastError();
}
