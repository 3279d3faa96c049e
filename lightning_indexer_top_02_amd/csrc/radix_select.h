// radix_select.h -- workgroup-level pieces of the radix Top-K selection.
//
// Keys are the order-preserving 32-bit images of fp32 scores (score_key), so
// "K largest scores" is "K largest keys".  The K-th largest key is found one
// radix digit at a time (11, 11 and 10 bits from the top): a histogram of the
// current digit over the keys that match the digits found so far, then a
// scan from the top bin down to the bin where the running count reaches the
// number of keys still needed.
#pragma once

#include "dsa_device.h"

namespace dsa {

constexpr int kLevelShift[3] = {21, 10, 0};   // low bit of each digit
constexpr int kLevelBins[3] = {2048, 2048, 1024};

// Largest bin `bin` with (keys in bins >= bin) >= k; above = keys in bins > bin;
// total = keys in all bins.  Run by one full wave (64 lanes); every lane
// returns the result.  Lane l reads its PER = nbins / 64 bins (the top ones
// for lane 0) with 16-byte LDS loads, so the bins are read once, in parallel.
// If the bins hold fewer than k keys it returns bin 0, above 0.
template <int PER>
__device__ __forceinline__ void load_bins_wave(const uint32_t* bins, uint32_t (&v)[PER]) {
  constexpr int nbins = PER * 64;
  const int lo = nbins - ((threadIdx.x & 63) + 1) * PER;  // lane owns bins [lo, lo + PER)
#pragma unroll
  for (int j = 0; j < PER; j += 4) {
    const uint4 q = *reinterpret_cast<const uint4*>(bins + lo + j);
    v[j] = q.x;
    v[j + 1] = q.y;
    v[j + 2] = q.z;
    v[j + 3] = q.w;
  }
}

// kth_bin_wave on bins a wave has already read with load_bins_wave.
template <int PER>
__device__ __forceinline__ void kth_bin_loaded(const uint32_t (&v)[PER], int k, int& bin, int& above, int& total) {
  constexpr int nbins = PER * 64;
  const int lane = threadIdx.x & 63;
  const int lo = nbins - (lane + 1) * PER;
  int local = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) local += (int)v[j];
  const int incl = wave_incl_scan(local);
  total = wave_read_lane(incl, 63);
  const int before = incl - local;
  // the lane whose bins cross k walks them from the top; selects with
  // constant j keep the walk free of per-bin registers and branches
  int fj = -1, ra = 0;
  if (before < k && incl >= k) {
    int acc = before;
#pragma unroll
    for (int j = PER - 1; j >= 0; --j) {
      const bool hit = fj < 0 && acc + (int)v[j] >= k;
      fj = hit ? j : fj;
      ra = hit ? acc : ra;
      acc += (int)v[j];
    }
  }
  const int rb = fj >= 0 ? lo + fj : -1;
  const uint64_t found = __ballot(rb >= 0);
  if (found == 0) {
    bin = 0;
    above = 0;
    return;
  }
  const int src = __ffsll((long long)found) - 1;
  bin = wave_read_lane(rb, src);
  above = wave_read_lane(ra, src);
}

// kth_bin_loaded that also returns the count of the bin it finds (0 when
// the bins hold fewer than k keys).
template <int PER>
__device__ __forceinline__ void kth_bin_wave_count(const uint32_t* bins, int k, int& bin, int& above, int& total,
                                                   int& count) {
  uint32_t v[PER];
  load_bins_wave<PER>(bins, v);
  kth_bin_loaded<PER>(v, k, bin, above, total);
  // the lane owning the bin reads its count
  const int lane = threadIdx.x & 63, lo = PER * 64 - (lane + 1) * PER;
  int mine = -1;
#pragma unroll
  for (int j = 0; j < PER; ++j) mine = lo + j == bin ? (int)v[j] : mine;
  const uint64_t owner = __ballot(mine >= 0);
  count = owner ? wave_read_lane(mine, __ffsll((long long)owner) - 1) : 0;
}

template <int PER>
__device__ __forceinline__ void kth_bin_wave(const uint32_t* bins, int k, int& bin, int& above, int& total) {
  uint32_t v[PER];
  load_bins_wave<PER>(bins, v);
  kth_bin_loaded<PER>(v, k, bin, above, total);
}

__device__ __forceinline__ void kth_bin_wave(const uint32_t* bins, int nbins, int k, int& bin, int& above) {
  int total;
  if (nbins == 2048) kth_bin_wave<32>(bins, k, bin, above, total);
  else kth_bin_wave<16>(bins, k, bin, above, total);
}

// Exclusive prefix sum of v over a workgroup of NT threads in thread order.
// `wsum` is LDS scratch of NT/64 ints (16-byte aligned).  Contains two barriers.
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, int& total, int* wsum) {
  constexpr int NW = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(v);
  __syncthreads();
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int ws[NW];
  if constexpr (NW % 4 == 0) {
#pragma unroll
    for (int w = 0; w < NW; w += 4) {
      const int4 q = *reinterpret_cast<const int4*>(wsum + w);
      ws[w] = q.x;
      ws[w + 1] = q.y;
      ws[w + 2] = q.z;
      ws[w + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int w = 0; w < NW; ++w) ws[w] = wsum[w];
  }
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    base += w < wave ? ws[w] : 0;
    total += ws[w];
  }
  return base + incl - v;
}

}  // namespace dsa

namespace dsa {

// Top-K of one row of `vis` <= NT * KPT keys held in registers, written to
// out[0..K) in ascending position order; ties at the K-th key go to the lower
// positions (rows with vis <= K are the caller's business).  The first digit
// is already known: bin1 is the top-11-bit bin of the K-th key (from a
// histogram of the whole row built elsewhere) and `need` the number of keys
// still to take from it.
//
// Layout: thread t holds key[c] = key of position KPT * t + c, so position
// order is thread order.  Slots at or past `vis` must hold key 0, which lies
// below the key of every finite score, so it is never above, equal to or at
// the K-th key of a row with vis > K.
//
// The two remaining digits (11 and 10 bits) come from LDS histograms
// (`hist`, kHistBins words) of the keys matching the digits found so far.
// When the second digit's bin holds exactly the keys still needed, all of
// them are kept whatever their low 10 bits, so the third digit is skipped
// and the keys are compared on their top 22 bits (the kept set is the same:
// every key of that bin is at or above the K-th).  With continuous scores
// that bin usually holds one key.
// Output: the kept keys are the keys above the K-th plus the first `need`
// keys equal to it.  Each thread builds bit masks of its keys above and equal
// to the K-th; one scan of the per-thread counts gives every thread its
// output offset, above_before + min(equal_before, need), and the thread
// writes the positions of its mask bits in order.  `wsum` holds NT / 64
// ints, `res` 3.
template <int NT, int KPT>
__device__ void select_from_level1(const uint32_t (&key)[KPT], int vis, int K, uint32_t bin1, int need,
                                   int32_t* out, uint32_t* hist, int* wsum, int* res) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int base = tid * KPT;
  const bool active = base < vis;
  uint32_t prefix = bin1;
  int low = 0;  // low key bits left unresolved (10 when the third digit is skipped)
  for (int level = 1; level < 3; ++level) {
    const int nbins = kLevelBins[level], shift = kLevelShift[level], pshift = kLevelShift[level - 1];
    for (int c = tid; c < nbins; c += NT) hist[c] = 0u;
    __syncthreads();
    if (active) {
#pragma unroll
      for (int c = 0; c < KPT; ++c) {
        const uint32_t k = key[c];
        if ((k >> pshift) == prefix) atomicAdd(&hist[(k >> shift) & (uint32_t)(nbins - 1)], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      int bin, above, total, count = -1;
      if (level == 1) kth_bin_wave_count<kLevelBins[1] / 64>(hist, need, bin, above, total, count);
      else kth_bin_wave<kLevelBins[2] / 64>(hist, need, bin, above, total);
      if (lane == 0) {
        res[0] = bin;
        res[1] = above;
        res[2] = count;
      }
    }
    __syncthreads();
    prefix = (prefix << (level == 1 ? 11 : 10)) | (uint32_t)res[0];
    need -= res[1];
    const bool whole = res[2] == need;  // (uniform: read from LDS by every thread)
    __syncthreads();
    if (whole) {
      low = shift;
      break;
    }
  }
  static_assert(KPT <= 32, "one mask bit per key");
  // the K-th key (its top 32 - low bits); a padding key 0 stays below it
  const uint32_t kth = prefix;
  uint32_t gtm = 0u, eqm = 0u;
#pragma unroll
  for (int c = 0; c < KPT; ++c) {
    const uint32_t k = key[c] >> low;
    gtm |= k > kth ? (1u << c) : 0u;
    eqm |= k == kth ? (1u << c) : 0u;
  }
  int packed_total;
  const int packed_before = block_excl_scan<NT>(__popc(gtm) | (__popc(eqm) << 16), packed_total, wsum);
  const int gt_before = packed_before & 0xffff, eq_before = packed_before >> 16;
  // the first (need - eq_before) of this thread's keys equal to the K-th stay
  uint32_t sel = gtm, e = eqm;
  for (int take = need - eq_before; take > 0 && e != 0u; --take) {
    sel |= e & (0u - e);
    e &= e - 1u;
  }
  int o = gt_before + min(eq_before, need);
  while (sel != 0u) {
    const int c = __builtin_ctz(sel);
    if (o < K) out[o] = base + c;
    ++o;
    sel &= sel - 1u;
  }
  __syncthreads();
}

}  // namespace dsa
