// sfa.hip -- sparse flash attention over the selected latent rows (gfx950).
//
// Phase 2 of the DSA step reads only the cache rows of the selected positions
// and attends over them ("Optimizing Inference for Hybrid Attention
// Architectures: From Operator Fusion to Sequence Sharding", section
// "Breaking Down the Computational Path of Hybrid Attention", item 2; "Day0
// Inference Support and Performance Optimization for New LLM Architectures",
// section III, 3.2).  The cache is the MLA latent cache: one shared 576-wide
// row per position (512 latent + 64 rope) used whole as the key and by its
// first 512 entries as the value.
//
// bf16 kernel (sfa_bf16): a workgroup owns one query row, 16 NW heads, and
// one contiguous slice of the row's index list.  The slice's pool rows are
// looked up through the block table once; the rows are then gathered in
// chunks of 32 into LDS (the scattered reads become 1152-byte row reads,
// "aggregating random small reads", "Optimizing Inference for Hybrid
// Attention LLMs: Practices for Fast Adaptation", section 3, item 2): while
// chunk c is computed from one LDS buffer, chunk c + 1 is written into the
// other and chunk c + 2's loads are in flight in registers (the same page's
// "overlapping gather and compute").  Each 16-head
// tile has two waves: per chunk, each computes S^T = K Q^T for half of the
// chunk's rows (16 rows x 16 heads, contraction 576) with MFMA, the two
// exchange their row maxima and probabilities through LDS, and each
// accumulates O^T += V^T P^T for half of the value dims (256 dims x 16
// heads, contraction over the 32 rows).  Computing the transposed products
// keeps each head's softmax state in one lane column, so the probabilities
// feed the second product straight from the first's accumulators.  When the
// index list is split over several workgroups (small batches), each writes a
// normalised partial output (fp16) and its log-sum-exp, and sfa_combine merges
// them.
//
// The tiles per workgroup (NW) follow the batch: one tile when the batch is
// at most 8 tiles, two up to 32, else four (see the host planner); absent
// rows and unneeded pieces read a zero row, so every gather load is issued.
//
// fp32 kernel (sfa_f32): VALU, one workgroup per (query row, 16 heads, split
// of the index list), merged by sfa_combine like the bf16 route.
#include <algorithm>

#include "dsa_device.h"

namespace dsa {

struct SfaParams {
  const int32_t* q_offsets;
  const int32_t* bt;
  int batch, bt_stride;
  int T, H;
  float scale;
  const void* q;
  const void* kv;
  const int32_t* idx;
  int K;
  void* out;
  float* lse;
  int n_split, rows_per_split;
  uint16_t* part_o;  // fp16
  float* part_lse;
};

constexpr int kSfaRows = 32;                 // rows per staged chunk
constexpr int kRowBytes = kQkDim * 2;        // 1152 bytes of bf16
constexpr int kRowStride = kRowBytes + 32;   // padded LDS row: 296 dwords, 40 mod 64 banks
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kRescale = 8.f;  // log2 headroom before the running maximum is moved

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even bf16 and packed (lo in the low
// half) by gfx950's one-instruction conversion, v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Split partials are stored as fp16 (nearest even): a normalised partial
// output is a convex combination of value elements, so its magnitude stays
// that of the values, and fp16's 11-bit significand keeps its rounding well
// inside the output tolerance (bf16's 8 bits did not: two roundings reached
// 2.4e-2 on integer-valued inputs), at half the bytes of fp32.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), f16x2_t));
}
// Two bf16 values scaled by a (to fp32 and back, round to nearest even).
__device__ __forceinline__ uint32_t scale_bf16x2(uint32_t v, float a) {
  return pack_bf16x2(__uint_as_float(v << 16) * a, __uint_as_float(v & 0xffff0000u) * a);
}

__device__ __forceinline__ float4 unpack_f16x4(uint2 v) {
  const f16x2_t a = __builtin_bit_cast(f16x2_t, v.x), b = __builtin_bit_cast(f16x2_t, v.y);
  return make_float4((float)a[0], (float)a[1], (float)b[0], (float)b[1]);
}

// LDS layout of one staged chunk of 32 rows: krow, a row-major copy of the
// whole 576-wide rows.  It is the A operand of S^T = K Q^T as it is, and
// gives the A operand of O^T += V^T P^T through gfx950's transposing LDS read
// (ds_read_b64_tr_b16): within each 16-lane group, lane L supplies 4
// consecutive 16-bit elements and lane i receives the i-th column of the 4 x
// 16 block the group supplied.  A lane of lane group g needs V^T[dim][slots
// 8g .. 8g + 7], where slot 8g + e holds row 4g + e (e < 4, the first half's
// S rows) or 16 + 4g + e - 4 (e >= 4, the second half's): the rows whose
// probabilities the lane holds, so P^T is the B operand as it comes out of
// the softmax.  Two transposing reads of rows 4g .. 4g + 3 and 16 + 4g ..
// 16 + 4g + 3 give those 8 elements.
// Bank spread (64 banks of 4 bytes): rows are 1184 bytes apart (40 mod 64
// banks), so the 8 rows a transposing read touches in one pass start 8 banks
// apart and fill all 64 (a 1168-byte stride left them overlapping, which
// measured 12 % slower).

constexpr int kKrowBytes = kSfaRows * kRowStride;

// Zeros standing in for an absent row (index -1, or a rope piece a lane does
// not load): every gather load is issued, from this row when there is
// nothing to read, so no branch surrounds a load and the waits for a chunk
// count exactly.  An fp8 row of zeros (codes and exponent bytes 0) decodes
// to zeros too.  (A global, not a constant-space, array: a pointer chosen
// between it and the pool stays a global pointer, so the loads stay global
// loads.  Nothing writes it.)
__device__ __align__(16) unsigned char kZeroRow[kRowBytes] = {};
// pointers into global memory (pool rows or the zero row), so the loads are
// global loads and cannot alias the gather registers
typedef const __attribute__((address_space(1))) unsigned char* gbyte_ptr;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 gload16(gbyte_ptr p) {
  return __builtin_bit_cast(uint4, *reinterpret_cast<const __attribute__((address_space(1))) u32x4_t*>(p));
}
constexpr int kPieces = kSfaRows * (kRowBytes / 16);  // 16-byte pieces of a chunk

// fp8 latent rows in HBM ("Day0 Inference Optimization for Next-Generation
// Hybrid-Architecture LLMs Based on CANN", section 3.2: an fp8 KV cache with
// a scale per token and 128-element tile): the 512 latent dims as e4m3 codes,
// a 16-byte block whose first four bytes are the tiles' E8M0 exponents
// (power-of-two scales), then the 64 rope dims in bf16, 656 bytes.  A chunk
// is gathered by 16 threads per row: thread k takes code pieces k and k + 16
// (16 codes each) and rope piece k (the zero row for k >= 8), and each of the
// 16 loads the row's exponent word (one address, so one cache line for the
// group).  The rows are staged in the same bf16 LDS layout as the
// bf16 route, so everything after the staging is shared.  code * 2^e is exact in
// bf16, and gfx950's scaled conversion (v_cvt_scalef32_pk_bf16_fp8, which
// applies the exponent of its fp32 scale operand) makes two values per
// instruction.
constexpr int kF8RowBytes = kVDim + 16 + 2 * (kQkDim - kVDim);
static_assert(kF8RowBytes % 16 == 0, "fp8 latent rows stay 16-byte aligned");

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 4 value elements of rows r0 .. r0 + 3 at one dim, per lane: see above.
__device__ __forceinline__ uint2 read_vt4(const unsigned char* krow, int r0, int d0) {
  const int L = threadIdx.x & 15;
  const unsigned char* a = krow + (r0 + (L >> 2)) * kRowStride + (d0 + 4 * (L & 3)) * 2;
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_v4i16*)(__attribute__((address_space(3))) unsigned char*)a);
  return __builtin_bit_cast(uint2, v);
}

// Exchange area between the two waves of a head tile (LDS, after the chunk
// buffers): the chunk maxima of each half's 16 rows, the probabilities each
// half feeds the other's P.V, and the final sums.  Sized for the workgroup's
// NW tiles, so a one-tile workgroup takes 79 KB of LDS with a 512-row split
// and two fit on a compute unit.
template <int NW>
struct SfaXchg {
  float tmax[2][NW][16];   // [half][head tile][head]
  uint2 pv[2][NW][64];     // [half][head tile][lane]: 4 bf16 probabilities
  float lsum[2][NW][16];   // [half][head tile][head]
};

// dynamic LDS of a bf16/fp8 workgroup: two chunk buffers, the exchange area
// and the split's row table
__host__ __device__ constexpr size_t sfa_lds_bytes(int nw, int rows_per_split) {
  return (size_t)2 * kKrowBytes + (size_t)nw * (2 * 16 * 4 + 2 * 64 * 8 + 2 * 16 * 4) +
         (size_t)(rows_per_split + kSfaRows - 1) / kSfaRows * kSfaRows * 4;
}

template <int NW, bool F8, bool TWO>
__global__ __launch_bounds__(NW * 128) void sfa_bf16(SfaParams p) {
  static_assert(!TWO || (NW == 1 && !F8), "two gather register sets: one-tile bf16 workgroups only");
  constexpr int NT = NW * 128;
  // fp8: RP rows per pass of 16 threads each, PASSES passes per chunk
  constexpr int RP = NT / 16, PASSES = (kSfaRows + RP - 1) / RP;
  constexpr int PPT = F8 ? 3 * PASSES : (kPieces + NT - 1) / NT;  // gathered pieces per thread per chunk
  constexpr int kHalfDims = kVDim / 2;
  extern __shared__ __align__(16) unsigned char smem[];
  static_assert(sizeof(SfaXchg<NW>) == (size_t)NW * (2 * 16 * 4 + 2 * 64 * 8 + 2 * 16 * 4), "sfa_lds_bytes");
  SfaXchg<NW>* xc = reinterpret_cast<SfaXchg<NW>*>(smem + 2 * kKrowBytes);
  int* rowidx = reinterpret_cast<int*>(smem + 2 * kKrowBytes + sizeof(SfaXchg<NW>));  // pool row, -1 = none

  // XCD-aware order: consecutive workgroups go to the eight XCDs in turn,
  // so the head groups of one (split, row) are given ids 8 apart and land on
  // one XCD, where the later ones find the gathered rows in its L2
  const int n_hg = p.H / (16 * NW);
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int hg = slot % n_hg;
  const int rs = (slot / n_hg) * 8 + xcd;  // (split, row) pair
  if (rs >= p.n_split * p.T) return;
  const int split = rs % p.n_split, i = rs / p.n_split;
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  // wave = (half, head tile): the tile's 16 heads; S for rows 16 half .. +16 of
  // each chunk, P.V for value dims 256 half .. +256
  const int ht = wave % NW, half = wave / NW;
  const int h = hg * (16 * NW) + ht * 16 + l16;  // this lane's head column
  const int r_begin = split * p.rows_per_split;
  const int nrows = max(0, min(p.K, r_begin + p.rows_per_split) - r_begin);
  const uint16_t* kvg = static_cast<const uint16_t*>(p.kv);

  // pool rows of this split's selected rows (index -> page -> slot), once
  {
    const int32_t* irow = p.idx + (int64_t)i * p.K + r_begin;
    const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
    const int nr = (nrows + kSfaRows - 1) / kSfaRows * kSfaRows;
    for (int r = tid; r < nr; r += NT) {
      const int t = r < nrows ? irow[r] : -1;
      rowidx[r] = t >= 0 ? btrow[t >> 6] * kPage + (t & 63) : -1;
    }
  }
  // Q fragments of this lane's head: qf[s] = q[h][32 s + 8 g .. + 8]
  uint4 qf[kQkDim / 32];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)i * p.H + h) * kQkDim;
#pragma unroll
    for (int s2 = 0; s2 < kQkDim / 32; ++s2) qf[s2] = *reinterpret_cast<const uint4*>(qrow + s2 * 32 + g * 8);
  }
  f32x4 o[kHalfDims / 16];
#pragma unroll
  for (int et = 0; et < kHalfDims / 16; ++et) o[et] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  const float zscale = p.scale * kLog2e;
  __syncthreads();

  // gather of one chunk into registers: PPT 16-byte pieces of its rows
  // (fp8: per pass two code pieces and a rope piece of one row, and the
  // row's exponent word on the first lane of each 16-lane group)
  uint4 va[PPT];
  uint32_t ew[F8 ? PASSES : 1];
  const unsigned char* kv8 = static_cast<const unsigned char*>(p.kv);
  auto gather_into = [&](uint4 (&va)[PPT], uint32_t (&ew)[F8 ? PASSES : 1], int c0) __attribute__((always_inline)) {
    if constexpr (F8) {
      const int k = tid & 15;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int r = ps * RP + (tid >> 4);
        const int row = r < kSfaRows ? rowidx[c0 + r] : -1;
        const gbyte_ptr zero = (gbyte_ptr)kZeroRow;
        const gbyte_ptr rb = row >= 0 ? (gbyte_ptr)(kv8 + (int64_t)row * kF8RowBytes) : zero;
        const gbyte_ptr rope = row >= 0 && k < 8 ? rb + kVDim + 16 + 16 * k : zero;
        va[3 * ps] = gload16(rb + 16 * k);
        va[3 * ps + 1] = gload16(rb + 16 * (k + 16));
        va[3 * ps + 2] = gload16(rope);
        ew[ps] = *reinterpret_cast<const __attribute__((address_space(1))) uint32_t*>(rb + kVDim);  // (one address per 16 lanes)
      }
    } else {
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        const int it = tid + j * NT;
        const int r = it / (kRowBytes / 16), part = it - r * (kRowBytes / 16);
        const int row = it < kPieces ? rowidx[c0 + r] : -1;
        const gbyte_ptr src = row >= 0 ? (gbyte_ptr)(kvg + (int64_t)row * kQkDim) : (gbyte_ptr)kZeroRow;
        va[j] = gload16(src + part * 16);
      }
    }
  };
  auto stage_from = [&](const uint4 (&va)[PPT], const uint32_t (&ew)[F8 ? PASSES : 1], unsigned char* kb)
                        __attribute__((always_inline)) {
    if constexpr (F8) {
      const int k = tid & 15;
#pragma unroll
      for (int ps = 0; ps < PASSES; ++ps) {
        const int r = ps * RP + (tid >> 4);
        const uint32_t e = ew[ps];  // the row's exponent word (every lane of the 16 loaded it)
        if (r >= kSfaRows) continue;
#pragma unroll
        for (int q = 0; q < 2; ++q) {  // code piece k + 16 q: 16 codes -> 16 bf16 values (32 bytes)
          const int piece = k + 16 * q;
          // the tile's scale 2^(E - 127) as an fp32 (exponent field E, E in 1 .. 254)
          const float sc = __uint_as_float(((e >> (8 * (piece >> 3))) & 0xFFu) << 23);
          const uint4 c = va[3 * ps + q];
          const uint32_t w[4] = {c.x, c.y, c.z, c.w};
          uint32_t o8[8];
#pragma unroll
          for (int m = 0; m < 4; ++m) {  // codes 4m, 4m + 1 (low half), 4m + 2, 4m + 3 (high half)
            o8[2 * m] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[m], sc, false));
            o8[2 * m + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[m], sc, true));
          }
          uint4* d = reinterpret_cast<uint4*>(kb + r * kRowStride + piece * 32);
          d[0] = make_uint4(o8[0], o8[1], o8[2], o8[3]);
          d[1] = make_uint4(o8[4], o8[5], o8[6], o8[7]);
        }
        if (k < 8)  // rope: already bf16
          *reinterpret_cast<uint4*>(kb + r * kRowStride + kVDim * 2 + 16 * k) = va[3 * ps + 2];
      }
    } else {
#pragma unroll
      for (int j = 0; j < PPT; ++j) {
        const int it = tid + j * NT;
        const int r = it / (kRowBytes / 16), part = it - r * (kRowBytes / 16);
        if (it < kPieces) *reinterpret_cast<uint4*>(kb + r * kRowStride + part * 16) = va[j];
      }
    }
  };

  // Two chunk buffers: chunk c is read from buffer c % 2 while chunk c + 1
  // is written into the other (after this chunk's S^T) and chunk c + 2's
  // loads are issued.  With TWO (one-tile bf16 workgroups whose split is one
  // or two chunks: the single-row decode) the gather uses two register sets
  // in turn, chunk c in set c % 2, so both chunks' loads are issued before
  // the first is staged (and on longer splits chunk c + 3's loads start as
  // chunk c + 1 is staged).  Measured: 16.5 against 16.8 us at the 32K
  // single-row decode; on 16-chunk splits (the 16-head batch of 64 rows)
  // two sets took 58.7 us against 53.0, and with fp8 rows 48.9 against 36.5.
  uint4 vb[TWO ? PPT : 1];
  uint32_t ewb[F8 ? PASSES : 1];
  auto gather = [&](int c0) __attribute__((always_inline)) { gather_into(va, ew, c0); };
  auto stage = [&](unsigned char* kb) __attribute__((always_inline)) { stage_from(va, ew, kb); };
  if (nrows > 0) {
    gather(0);
    if constexpr (TWO) {
      if (nrows > kSfaRows) gather_into(vb, ewb, kSfaRows);
      __builtin_amdgcn_sched_barrier(0);  // (both sets' loads are issued before the staging waits)
    }
    stage(smem);
  }
  if (nrows > kSfaRows) {
    if constexpr (TWO) {
      if (nrows > 2 * kSfaRows) gather(2 * kSfaRows);
    } else {
      gather(kSfaRows);
    }
  }
  for (int c0 = 0; c0 < nrows; c0 += kSfaRows) {
    __syncthreads();  // chunk c is staged; the other buffer (chunk c - 1) is no longer read
    const unsigned char* krow = smem + ((c0 / kSfaRows) & 1) * kKrowBytes;

    // S^T tile of this half: s[e] = S[head l16][row 16 half + 4g + e]; two
    // accumulators (even and odd contraction steps) halve the dependent chain
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* ka = krow + (16 * half + l16) * kRowStride + g * 16;
#pragma unroll
    for (int s2 = 0; s2 < kQkDim / 32; s2 += 2) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(ka + s2 * 64);
      const uint4 a1 = *reinterpret_cast<const uint4*>(ka + (s2 + 1) * 64);
      sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qf[s2]), sa, 0, 0, 0);
      sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qf[s2 + 1]), sb, 0, 0, 0);
    }
    sa += sb;
    if (c0 + kSfaRows < nrows) {
      unsigned char* kb = smem + (((c0 / kSfaRows) + 1) & 1) * kKrowBytes;
      if constexpr (TWO) {
        // chunk c + 1 is in set (c + 1) % 2; chunk c + 3 goes into it next
        if (((c0 / kSfaRows) & 1) == 0) {
          stage_from(vb, ewb, kb);
          if (c0 + 3 * kSfaRows < nrows) gather_into(vb, ewb, c0 + 3 * kSfaRows);
        } else {
          stage(kb);
          if (c0 + 3 * kSfaRows < nrows) gather(c0 + 3 * kSfaRows);
        }
      } else {
        stage(kb);
        if (c0 + 2 * kSfaRows < nrows) gather(c0 + 2 * kSfaRows);
      }
    }
    float z[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) z[e] = rowidx[c0 + 16 * half + 4 * g + e] >= 0 ? sa[e] * zscale : -INFINITY;
    float tmax = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
    tmax = group4_max(tmax);  // this half's chunk maximum per head
    // Lazy rescaling: the reference maximum m only moves when some head's
    // chunk maximum exceeds it by more than 2^kRescale (the exponentials stay
    // <= 2^kRescale otherwise, well inside fp32 and bf16), and then for the
    // whole wave, so most chunks skip the pass over the accumulators.
    //   TWO (the single-row decode, two chunks a split): the halves first
    //   exchange their chunk maxima and take the same decision from the same
    //   values (one more barrier, measured 0.07 us faster there).
    //   Otherwise each half decides from its own rows and the two references
    //   are brought together after the probability exchange.  References are
    //   then whole numbers (log2 units), so every rescaling factor is a power
    //   of two and rescales bf16 probabilities and the accumulators exactly
    //   (prefill 3.47 against 3.60 ms, 64-row decode 70.8 against 72.1 us).
    if constexpr (TWO) {
      if (g == 0) xc->tmax[half][ht][l16] = tmax;
      __syncthreads();
      tmax = fmaxf(tmax, xc->tmax[half ^ 1][ht][l16]);  // the chunk's maximum, the same in both halves
    }
    if (__ballot(tmax > m + kRescale)) {
      const float mnew = TWO ? fmaxf(m, tmax) : ceilf(fmaxf(m, tmax));
      if (__ballot(m != -INFINITY)) {  // (all zero before the first rows)
        const float alpha = exp2f(m - mnew);
        lsum *= alpha;
#pragma unroll
        for (int et = 0; et < kHalfDims / 16; ++et) o[et] *= alpha;
      }
      m = mnew;
    }
    // exponentials with the bare hardware exp2 (v_exp_f32: exp2(-inf) = 0,
    // results below 2^-126 flush to 0, far below the row's largest term, 1);
    // m is -inf only while every row so far has been padding
    const float mref = m == -INFINITY ? 0.f : m;
    float pr[4], psum = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pr[e] = __builtin_amdgcn_exp2f(z[e] - mref);
      psum += pr[e];
    }
    lsum += group4_sum(psum);  // this half's rows only; the halves are added at the end
    uint2 mine;
    mine.x = pack_bf16x2(pr[0], pr[1]);
    mine.y = pack_bf16x2(pr[2], pr[3]);
    xc->pv[half][ht][lane] = mine;
    if (!TWO && g == 0) xc->tmax[half][ht][l16] = m;  // the reference these probabilities are relative to
    __syncthreads();
    uint2 other = xc->pv[half ^ 1][ht][lane];
    if constexpr (!TWO) {
      const float mo = xc->tmax[half ^ 1][ht][l16];
      if (__ballot(mo != m)) {  // the halves moved their references differently: both go to the larger (exact)
        const float mc = fmaxf(m, mo);
        const float am = m == mc ? 1.f : exp2f(m - mc), ao = mo == mc ? 1.f : exp2f(mo - mc);
        lsum *= am;
#pragma unroll
        for (int et = 0; et < kHalfDims / 16; ++et) o[et] *= am;
        mine.x = scale_bf16x2(mine.x, am);
        mine.y = scale_bf16x2(mine.y, am);
        other.x = scale_bf16x2(other.x, ao);
        other.y = scale_bf16x2(other.y, ao);
        m = mc;
      }
    }
    // B operand of O^T += V^T P^T in slot order: rows 4g + e (half 0), then 16 + 4g + e (half 1)
    uint4 pf;
    pf.x = half ? other.x : mine.x;
    pf.y = half ? other.y : mine.y;
    pf.z = half ? mine.x : other.x;
    pf.w = half ? mine.y : other.y;
#pragma unroll
    for (int et = 0; et < kHalfDims / 16; ++et) {
      const int d0 = kHalfDims * half + 16 * et;
      const uint2 lo = read_vt4(krow, 4 * g, d0), hi = read_vt4(krow, 16 + 4 * g, d0);
      const uint4 av = make_uint4(lo.x, lo.y, hi.x, hi.y);
      o[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(pf), o[et], 0, 0, 0);
    }
  }

  // both halves' row sums (the same m in both)
  if (g == 0) xc->lsum[half][ht][l16] = lsum;
  __syncthreads();
  lsum = half ? xc->lsum[0][ht][l16] + lsum : lsum + xc->lsum[1][ht][l16];
  // o[et][e] = unnormalised output of head h at dim 256 half + 16 et + 4 g + e
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float lse_v = lsum > 0.f ? m * kLn2 + logf(lsum) : -INFINITY;
  const int d0 = kHalfDims * half + 4 * g;
  if (p.n_split == 1) {
    uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)i * p.H + h) * kVDim + d0;
#pragma unroll
    for (int et = 0; et < kHalfDims / 16; ++et) {
      uint2 v;
      v.x = pack_bf16x2(o[et][0] * inv, o[et][1] * inv);
      v.y = pack_bf16x2(o[et][2] * inv, o[et][3] * inv);
      *reinterpret_cast<uint2*>(orow + et * 16) = v;
    }
    if (p.lse && g == 0 && half == 0) p.lse[(int64_t)i * p.H + h] = lse_v;
  } else {
    uint16_t* prow = p.part_o + (((int64_t)split * p.T + i) * p.H + h) * kVDim + d0;
#pragma unroll
    for (int et = 0; et < kHalfDims / 16; ++et)
      *reinterpret_cast<uint2*>(prow + et * 16) =
          make_uint2(pack_f16x2(o[et][0] * inv, o[et][1] * inv), pack_f16x2(o[et][2] * inv, o[et][3] * inv));
    if (g == 0 && half == 0) p.part_lse[((int64_t)split * p.T + i) * p.H + h] = lse_v;
  }
}

// Merge split partials: out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
// G threads per (query row, head, 4 output dims), 128 G threads per head, so
// a decode row's merge is spread over the whole chip.  Thread g of a group
// takes splits g, g + G, ..., reading them 16 at a time with all their loads
// in flight and folding them in with a running maximum (the sum is rescaled
// when the maximum grows); the G partial merges are then combined across
// neighbouring lanes, lower lane first, so every lane of a group forms the
// same result.  With G = 4 a merge of up to 64 splits is one memory round
// trip (few rows, many splits); G = 1 keeps the grid small for large batches,
// and G = 2 sits between (8 to 31 splits).
// NB, the splits a thread reads at once, is the smallest of 2, 4, 8, 16 that
// covers its share, so a two-split merge computes no exponentials for
// absent splits (the sums are the same for any NB: an absent split adds 0).
constexpr int kCombineThreads = 256;

template <bool BF16, int G, int NB>
__global__ __launch_bounds__(kCombineThreads) void sfa_combine(SfaParams p) {
  static_assert(G == 1 || G == 2 || G == 4, "lane groups within a quad");
  const int64_t gt = (int64_t)blockIdx.x * kCombineThreads + threadIdx.x;
  const int sg = (int)(gt % G);
  const int64_t rest = gt / G;
  const int64_t th = rest >> 7;           // = i * H + h
  const int d0 = (int)(rest & 127) * 4;   // first of this group's 4 dims
  const int64_t stride = (int64_t)p.T * p.H;
  // (whole groups are in range or out of it: the grid is a multiple of G)
  const bool ok = th < stride;
  float M = -INFINITY, den = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const uint16_t* po = p.part_o + (ok ? th : 0) * kVDim + d0;
  for (int s0 = 0; ok && s0 * G < p.n_split; s0 += NB) {
    float l[NB];
    float4 o[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int s = (s0 + j) * G + sg;
      l[j] = s < p.n_split ? p.part_lse[s * stride + th] : -INFINITY;
      o[j] = s < p.n_split ? unpack_f16x4(*reinterpret_cast<const uint2*>(po + s * stride * kVDim))
                           : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float bm = l[0];
#pragma unroll
    for (int j = 1; j < NB; ++j) bm = fmaxf(bm, l[j]);
    if (bm == -INFINITY) continue;  // no selected rows in these splits
    const float Mn = fmaxf(M, bm);
    const float r = expf(M - Mn);   // M = -inf gives 0 (acc and den are 0 then)
    den *= r;
    acc.x *= r; acc.y *= r; acc.z *= r; acc.w *= r;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float wgt = l[j] == -INFINITY ? 0.f : expf(l[j] - Mn);
      den += wgt;
      acc.x += wgt * o[j].x; acc.y += wgt * o[j].y; acc.z += wgt * o[j].z; acc.w += wgt * o[j].w;
    }
    M = Mn;
  }
#pragma unroll
  for (int off = 1; off < G; off <<= 1) {  // (every lane of the wave is here)
    const float Mo = quad_xor(M, off), deno = quad_xor(den, off);
    const float4 acco = make_float4(quad_xor(acc.x, off), quad_xor(acc.y, off), quad_xor(acc.z, off),
                                    quad_xor(acc.w, off));
    const bool upper = (sg & off) != 0;  // this lane's partial goes second
    const float Ma = upper ? Mo : M, Mb = upper ? M : Mo;
    const float da = upper ? deno : den, db = upper ? den : deno;
    const float4 aa = upper ? acco : acc, ab = upper ? acc : acco;
    const float Mn = fmaxf(Ma, Mb);
    const float ra = Ma == -INFINITY ? 0.f : expf(Ma - Mn), rb = Mb == -INFINITY ? 0.f : expf(Mb - Mn);
    den = da * ra + db * rb;
    acc = make_float4(aa.x * ra + ab.x * rb, aa.y * ra + ab.y * rb, aa.z * ra + ab.z * rb, aa.w * ra + ab.w * rb);
    M = Mn;
  }
  if (!ok || sg != 0) return;
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if (BF16) {
    uint2 v;
    v.x = pack_bf16x2(acc.x * inv, acc.y * inv);
    v.y = pack_bf16x2(acc.z * inv, acc.w * inv);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + th * kVDim + d0) = v;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + th * kVDim + d0) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (p.lse && d0 == 0) p.lse[th] = den > 0.f ? M + logf(den) : -INFINITY;
}

// fp32 (VALU): one workgroup per (query row, 16 heads, split of the Top-K
// list), like the bf16 route, so a single-row decode spreads over the chip.
// The split's selected rows are staged 16 at a time in LDS (580-float rows:
// 580 = 4 mod 64 banks, so the 16 rows a wave reads at one dim fall in 16
// different bank groups); thread (h, r) forms the logit of head h and row r,
// an online softmax runs over the chunks, and each thread then owns two
// output dims of all 16 heads.  Splits write fp16 partials for sfa_combine;
// a single split writes the output.
constexpr int kF32Threads = 256;
constexpr int kF32Rows = 16;               // selected rows per chunk
constexpr int kF32Heads = 16;              // heads per workgroup
constexpr int kF32Stride = kQkDim + 4;     // padded LDS row (floats)
static_assert(kF32Rows * kF32Heads == kF32Threads, "one logit per thread");
static_assert(2 * kF32Threads == kVDim, "two output dims per thread");

__host__ __device__ constexpr size_t sfa_f32_lds(int rows_per_split) {
  return (size_t)(kF32Heads + kF32Rows) * kF32Stride * 4 + (size_t)(kF32Heads * kF32Rows + 2 * kF32Heads) * 4 +
         (size_t)(rows_per_split + kF32Rows - 1) / kF32Rows * kF32Rows * 4;
}

__global__ __launch_bounds__(kF32Threads) void sfa_f32(SfaParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  float* qs = reinterpret_cast<float*>(smem);                // [16 heads][kF32Stride]
  float* ks = qs + kF32Heads * kF32Stride;                   // [16 rows][kF32Stride]
  float* pz = ks + kF32Rows * kF32Stride;                    // [16 heads][16 rows] probabilities
  float* hs = pz + kF32Heads * kF32Rows;                     // [16] rescale factors, then [2][16] m and l
  int* rowidx = reinterpret_cast<int*>(hs + 2 * kF32Heads);  // pool row of each selected row, -1 = none
  const int n_hg = p.H / kF32Heads;
  const int hg = blockIdx.x % n_hg, rs = blockIdx.x / n_hg;
  const int split = rs % p.n_split, i = rs / p.n_split;
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int tid = threadIdx.x;
  const int r_begin = split * p.rows_per_split;
  const int nrows = max(0, min(p.K, r_begin + p.rows_per_split) - r_begin);
  const int nr = (nrows + kF32Rows - 1) / kF32Rows * kF32Rows;
  {
    const int32_t* irow = p.idx + (int64_t)i * p.K + r_begin;
    const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
    for (int r = tid; r < nr; r += kF32Threads) {
      const int t = r < nrows ? irow[r] : -1;
      rowidx[r] = t >= 0 ? btrow[t >> 6] * kPage + (t & 63) : -1;
    }
  }
  const float* qg = static_cast<const float*>(p.q) + ((int64_t)i * p.H + hg * kF32Heads) * kQkDim;
  for (int e = tid; e < kF32Heads * (kQkDim / 4); e += kF32Threads) {
    const int h = e / (kQkDim / 4), d4 = e - h * (kQkDim / 4);
    *reinterpret_cast<float4*>(qs + h * kF32Stride + 4 * d4) = reinterpret_cast<const float4*>(qg + h * kQkDim)[d4];
  }
  const float4* kv4 = static_cast<const float4*>(p.kv);
  const int h = tid >> 4, r = tid & 15;  // this thread's logit
  const int d0 = 2 * tid;                // this thread's output dims
  float m = -INFINITY, l = 0.f;          // head h's running maximum and sum (the same in its 16 lanes)
  float acc[kF32Heads][2];
#pragma unroll
  for (int hh = 0; hh < kF32Heads; ++hh) acc[hh][0] = acc[hh][1] = 0.f;
  for (int c0 = 0; c0 < nr; c0 += kF32Rows) {
    __syncthreads();  // rowidx and the Q tile written; the previous chunk's rows no longer read
    for (int e = tid; e < kF32Rows * (kQkDim / 4); e += kF32Threads) {
      const int rr = e / (kQkDim / 4), d4 = e - rr * (kQkDim / 4);
      const int row = rowidx[c0 + rr];
      *reinterpret_cast<float4*>(ks + rr * kF32Stride + 4 * d4) =
          row >= 0 ? kv4[(int64_t)row * (kQkDim / 4) + d4] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
    float dot = 0.f;
    const float4* q4 = reinterpret_cast<const float4*>(qs + h * kF32Stride);
    const float4* k4 = reinterpret_cast<const float4*>(ks + r * kF32Stride);
#pragma unroll 8
    for (int d4 = 0; d4 < kQkDim / 4; ++d4) {
      const float4 a = q4[d4], k = k4[d4];
      dot = fmaf(a.x, k.x, dot);
      dot = fmaf(a.y, k.y, dot);
      dot = fmaf(a.z, k.z, dot);
      dot = fmaf(a.w, k.w, dot);
    }
    const bool live = rowidx[c0 + r] >= 0;
    const float z = live ? dot * p.scale : -INFINITY;
    float cm = z;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));  // over head h's 16 lanes
    const float mn = fmaxf(m, cm);
    const float al = mn == -INFINITY ? 1.f : expf(m - mn);  // (m = -inf: 0)
    const float pr = live ? expf(z - mn) : 0.f;
    float ps = pr;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
    l = l * al + ps;
    m = mn;
    pz[h * kF32Rows + r] = pr;
    if (r == 0) hs[h] = al;
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < kF32Heads; ++hh) {
      const float a = hs[hh];
      acc[hh][0] *= a;
      acc[hh][1] *= a;
    }
#pragma unroll 4
    for (int rr = 0; rr < kF32Rows; ++rr) {
      const float2 v = *reinterpret_cast<const float2*>(ks + rr * kF32Stride + d0);
#pragma unroll
      for (int hh = 0; hh < kF32Heads; ++hh) {
        const float pv = pz[hh * kF32Rows + rr];
        acc[hh][0] = fmaf(pv, v.x, acc[hh][0]);
        acc[hh][1] = fmaf(pv, v.y, acc[hh][1]);
      }
    }
  }
  __syncthreads();  // the last chunk's factors read
  if (r == 0) {
    hs[h] = m;
    hs[kF32Heads + h] = l;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < kF32Heads; ++hh) {
    const float lh = hs[kF32Heads + hh];
    const float inv = lh > 0.f ? 1.f / lh : 0.f;
    const int64_t th = (int64_t)i * p.H + hg * kF32Heads + hh;
    if (p.n_split == 1)
      *reinterpret_cast<float2*>(static_cast<float*>(p.out) + th * kVDim + d0) =
          make_float2(acc[hh][0] * inv, acc[hh][1] * inv);
    else
      *reinterpret_cast<uint32_t*>(p.part_o + ((int64_t)split * p.T * p.H + th) * kVDim + d0) =
          pack_f16x2(acc[hh][0] * inv, acc[hh][1] * inv);
  }
  if (tid < kF32Heads) {
    const float lh = hs[kF32Heads + tid];
    const float lse_v = lh > 0.f ? hs[tid] + logf(lh) : -INFINITY;
    const int64_t th = (int64_t)i * p.H + hg * kF32Heads + tid;
    if (p.n_split == 1) {
      if (p.lse) p.lse[th] = lse_v;
    } else {
      p.part_lse[(int64_t)split * p.T * p.H + th] = lse_v;
    }
  }
}
}  // namespace dsa

using namespace dsa;

template <int NW, bool F8, bool TWO = false>
static hipError_t launch_sfa(dim3 grid, size_t lds, hipStream_t s, const SfaParams& p) {
  {
    const hipError_t e = dsa_allow_lds(reinterpret_cast<const void*>(sfa_bf16<NW, F8, TWO>), lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((sfa_bf16<NW, F8, TWO>), grid, dim3(NW * 128), lds, s, p);
  return hipGetLastError();
}

template <bool F8>
static hipError_t launch_sfa_nw(int nw, dim3 grid, size_t lds, hipStream_t s, const SfaParams& p) {
  switch (nw) {
    case 1:
      if constexpr (!F8)  // splits of at most two chunks: both gathered at once (see sfa_bf16)
        if (p.rows_per_split <= 2 * kSfaRows) return launch_sfa<1, false, true>(grid, lds, s, p);
      return launch_sfa<1, F8>(grid, lds, s, p);
    case 2: return launch_sfa<2, F8>(grid, lds, s, p);
    case 3: return launch_sfa<3, F8>(grid, lds, s, p);
    default: return launch_sfa<4, F8>(grid, lds, s, p);
  }
}

template <bool BF16>
static hipError_t launch_combine(const DsaSfaLaunch& a, hipStream_t s, const SfaParams& p) {
  const int64_t groups = (int64_t)a.num_rows * a.n_heads * (kVDim / 4);
  // lanes per (row, head, 4 dims): 4 for 32 splits and more, 2 for 8 to 31
  // (a batch-8 decode has 16: 26.2 us against 28.0 with 4), 1 below
  const int G = a.n_split >= 32 ? 4 : (a.n_split >= 8 ? 2 : 1);
  const int share = (a.n_split + G - 1) / G;  // splits per thread
  const dim3 cgrid((unsigned)((G * groups + kCombineThreads - 1) / kCombineThreads));
  if (G == 4) {
    if (share <= 2) hipLaunchKernelGGL((sfa_combine<BF16, 4, 2>), cgrid, dim3(kCombineThreads), 0, s, p);
    else if (share <= 4) hipLaunchKernelGGL((sfa_combine<BF16, 4, 4>), cgrid, dim3(kCombineThreads), 0, s, p);
    else if (share <= 8) hipLaunchKernelGGL((sfa_combine<BF16, 4, 8>), cgrid, dim3(kCombineThreads), 0, s, p);
    else hipLaunchKernelGGL((sfa_combine<BF16, 4, 16>), cgrid, dim3(kCombineThreads), 0, s, p);
  } else if (G == 2) {
    if (share <= 4) hipLaunchKernelGGL((sfa_combine<BF16, 2, 4>), cgrid, dim3(kCombineThreads), 0, s, p);
    else if (share <= 8) hipLaunchKernelGGL((sfa_combine<BF16, 2, 8>), cgrid, dim3(kCombineThreads), 0, s, p);
    else hipLaunchKernelGGL((sfa_combine<BF16, 2, 16>), cgrid, dim3(kCombineThreads), 0, s, p);
  } else {
    if (share <= 2) hipLaunchKernelGGL((sfa_combine<BF16, 1, 2>), cgrid, dim3(kCombineThreads), 0, s, p);
    else if (share <= 4) hipLaunchKernelGGL((sfa_combine<BF16, 1, 4>), cgrid, dim3(kCombineThreads), 0, s, p);
    else hipLaunchKernelGGL((sfa_combine<BF16, 1, 8>), cgrid, dim3(kCombineThreads), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t dsa_launch_sparse_attn(const DsaSfaLaunch& a, hipStream_t s) {
  SfaParams p;
  p.q_offsets = a.q_offsets;
  p.bt = a.block_table;
  p.batch = a.batch;
  p.bt_stride = a.bt_stride;
  p.T = a.num_rows;
  p.H = a.n_heads;
  p.scale = a.scale;
  p.q = a.q;
  p.kv = a.kv_cache;
  p.idx = a.idx;
  p.K = a.topk;
  p.out = a.out;
  p.lse = a.lse;
  p.n_split = a.n_split;
  p.rows_per_split = a.rows_per_split;
  p.part_o = a.part_o;
  p.part_lse = a.part_lse;
  if (a.dtype == 0) {
    if (a.n_heads % kF32Heads != 0) return hipErrorInvalidValue;
    const int64_t wgs = (int64_t)a.n_split * a.num_rows * (a.n_heads / kF32Heads);
    if (wgs * kF32Threads > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
    const size_t lds = sfa_f32_lds(a.rows_per_split);
    const hipError_t e0 = dsa_allow_lds(reinterpret_cast<const void*>(sfa_f32), lds);
    if (e0 != hipSuccess) return e0;
    hipLaunchKernelGGL(sfa_f32, dim3((unsigned)wgs), dim3(kF32Threads), lds, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.n_split == 1) return e;
    return launch_combine<false>(a, s, p);
  }
  const int nw = a.nw;  // 16-head tiles per workgroup
  if (nw < 1 || nw > 4 || (a.n_heads / 16) % nw != 0) return hipErrorInvalidValue;
  // one dimension: (split, row) pairs in groups of eight, each group's head
  // groups 8 workgroups apart (see sfa_bf16)
  const int64_t pairs = (int64_t)a.n_split * a.num_rows;
  const int64_t wgs = (pairs + 7) / 8 * 8 * (a.n_heads / (16 * nw));
  // the work-item count of one grid dimension has to fit 32 bits
  if (wgs * nw * 128 > (int64_t)UINT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)wgs);
  hipError_t e0;
  const size_t lds = sfa_lds_bytes(nw, a.rows_per_split);
  e0 = a.dtype == 2 ? launch_sfa_nw<true>(nw, grid, lds, s, p) : launch_sfa_nw<false>(nw, grid, lds, s, p);
  if (e0 != hipSuccess) return e0;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  return launch_combine<true>(a, s, p);
}
