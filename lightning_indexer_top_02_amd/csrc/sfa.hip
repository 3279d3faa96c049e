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
// bf16 kernel (sfa_bf16): a workgroup owns one query row, 16 heads per wave,
// and one contiguous slice of the row's index list.  The slice's pool rows
// are looked up through the block table once; the rows are then gathered in
// chunks of 32 into LDS (the scattered reads become 1152-byte row reads,
// "aggregating random small reads", "Optimizing Inference for Hybrid
// Attention LLMs: Practices for Fast Adaptation", section 3, item 2), the
// next chunk's loads in flight in registers while the current chunk is
// computed (the same page's "overlapping gather and compute"), and every wave
// of the workgroup reuses them.  Per chunk and wave, MFMA computes S^T = K Q^T (32 rows x 16 heads,
// contraction 576), an online softmax updates the running max and sum per
// head, and MFMA accumulates O^T += V^T P^T (512 dims x 16 heads,
// contraction over the 32 rows).  Computing the transposed products keeps
// each head's softmax state in one lane column, so the probabilities feed the
// second product straight from the first's accumulators.  When the index list
// is split over several workgroups (small batches), each writes a normalised
// partial output and its log-sum-exp, and sfa_combine merges them.
//
// fp32 kernel (sfa_f32): VALU, one workgroup per (query row, head).
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
  float* part_o;
  float* part_lse;
};

constexpr int kSfaRows = 32;                 // rows per staged chunk
constexpr int kRowBytes = kQkDim * 2;        // 1152 bytes of bf16
constexpr int kRowStride = kRowBytes + 16;   // padded LDS row (bank spread)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

// LDS layout of one staged chunk of 32 rows:
//   krow: row-major copy of the whole 576-wide rows (the A operand of
//         S^T = K Q^T), 1168-byte rows;
//   vt:   the value part (dims 0..511) transposed, vt[dim][slot], 80 bytes
//         per dim, where slot 8g + e holds row r(g, e) = 4g + e (e < 4) or
//         16 + 4g + e - 4 (e >= 4): the rows a lane of lane group g holds in
//         its S^T accumulators, so the probabilities are the B operand of
//         O^T += V^T P^T as they come out of the softmax and the A operand
//         is one 16-byte read.
//   The paddings make the MFMA operand reads and the staging writes
//   conflict-free (or at most 2-way) across the 64 LDS banks.
constexpr int kVtStride = 80;
constexpr int kKrowBytes = kSfaRows * kRowStride;
constexpr int kVtBytes = kVDim * kVtStride;

__device__ __forceinline__ int slot_row(int g, int e) { return e < 4 ? 4 * g + e : 16 + 4 * g + (e - 4); }

// Stage the 8 rows of lane group g (slot order), 8 value dims starting at
// dim 8 dc, into krow and (transposed) into vt.
__device__ __forceinline__ void stage_vblock(unsigned char* krow, unsigned char* vt, int g, int dc,
                                             const uint4 (&a)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e)
    *reinterpret_cast<uint4*>(krow + slot_row(g, e) * kRowStride + dc * 16) = a[e];
  // 8 x 8 transpose of 16-bit elements: t[j] holds dim 8 dc + j of the 8 rows
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = j >> 1;
    const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
    uint4 t;
    t.x = __builtin_amdgcn_perm(((const uint32_t*)&a[1])[k], ((const uint32_t*)&a[0])[k], sel);
    t.y = __builtin_amdgcn_perm(((const uint32_t*)&a[3])[k], ((const uint32_t*)&a[2])[k], sel);
    t.z = __builtin_amdgcn_perm(((const uint32_t*)&a[5])[k], ((const uint32_t*)&a[4])[k], sel);
    t.w = __builtin_amdgcn_perm(((const uint32_t*)&a[7])[k], ((const uint32_t*)&a[6])[k], sel);
    *reinterpret_cast<uint4*>(vt + (dc * 8 + j) * kVtStride + g * 16) = t;
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void sfa_bf16(SfaParams p) {
  constexpr int NT = NW * 64;
  constexpr int kBlocks = 4 * (kVDim / 8);              // (lane group, 8-dim chunk) blocks per chunk
  constexpr int kRope = kSfaRows * ((kQkDim - kVDim) / 8);  // 16-byte rope pieces per chunk
  constexpr int BPT = (kBlocks + NT - 1) / NT;            // value blocks per thread
  constexpr int RPT = (kRope + NT - 1) / NT;               // rope pieces per thread
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* krow = smem;
  unsigned char* vt = smem + kKrowBytes;
  int* rowidx = reinterpret_cast<int*>(smem + kKrowBytes + kVtBytes);  // pool row of each selected row, -1 = none

  const int split = blockIdx.x, hg = blockIdx.y, i = blockIdx.z;
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int h = hg * (16 * NW) + wave * 16 + l16;  // this lane's head column
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
  f32x4 o[kVDim / 16];
#pragma unroll
  for (int et = 0; et < kVDim / 16; ++et) o[et] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  const float zscale = p.scale * kLog2e;
  __syncthreads();

  // gather of one chunk into registers: BPT value blocks and RPT rope pieces
  uint4 va[BPT][8], ra[RPT];
  auto gather = [&](int c0) {
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int blk = tid + j * NT;
      const int gg = blk & 3, dc = blk >> 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = blk < kBlocks ? rowidx[c0 + slot_row(gg, e)] : -1;
        va[j][e] = row >= 0 ? *reinterpret_cast<const uint4*>(kvg + (int64_t)row * kQkDim + dc * 8)
                            : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int it = tid + j * NT;
      const int row = it < kRope ? rowidx[c0 + (it >> 3)] : -1;
      ra[j] = row >= 0 ? *reinterpret_cast<const uint4*>(kvg + (int64_t)row * kQkDim + kVDim + (it & 7) * 8)
                       : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int j = 0; j < BPT; ++j) {
      const int blk = tid + j * NT;
      if (blk < kBlocks) stage_vblock(krow, vt, blk & 3, blk >> 2, va[j]);
    }
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int it = tid + j * NT;
      if (it < kRope) *reinterpret_cast<uint4*>(krow + (it >> 3) * kRowStride + kVDim * 2 + (it & 7) * 16) = ra[j];
    }
  };

  if (nrows > 0) gather(0);
  for (int c0 = 0; c0 < nrows; c0 += kSfaRows) {
    __syncthreads();  // the previous chunk is no longer read
    stage();
    __syncthreads();
    if (c0 + kSfaRows < nrows) gather(c0 + kSfaRows);  // in flight during this chunk's math

    // S^T tiles: s0[e] = S[head l16][row 4g+e], s1[e] = S[head l16][row 16+4g+e]
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* ka = krow + l16 * kRowStride + g * 16;
#pragma unroll
    for (int s2 = 0; s2 < kQkDim / 32; ++s2) {
      const uint4 a0 = *reinterpret_cast<const uint4*>(ka + s2 * 64);
      const uint4 a1 = *reinterpret_cast<const uint4*>(ka + 16 * kRowStride + s2 * 64);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qf[s2]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qf[s2]), s1, 0, 0, 0);
    }
    float z[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = rowidx[c0 + 4 * g + e] >= 0 ? s0[e] * zscale : -INFINITY;
      z[4 + e] = rowidx[c0 + 16 + 4 * g + e] >= 0 ? s1[e] * zscale : -INFINITY;
    }
    float tmax = z[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, z[e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float mnew = fmaxf(m, tmax);
    float pr[8], alpha = 1.f, psum = 0.f;
    if (mnew == -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = 0.f;
    } else {
      alpha = exp2f(m - mnew);  // m = -inf gives 0
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pr[e] = exp2f(z[e] - mnew);
        psum += pr[e];
      }
    }
    psum += __shfl_xor(psum, 16);
    psum += __shfl_xor(psum, 32);
    lsum = lsum * alpha + psum;
    m = mnew;

    uint4 pf;  // B operand of O^T += V^T P^T, slot order
    pf.x = pack_bf16x2(pr[0], pr[1]);
    pf.y = pack_bf16x2(pr[2], pr[3]);
    pf.z = pack_bf16x2(pr[4], pr[5]);
    pf.w = pack_bf16x2(pr[6], pr[7]);
    const unsigned char* vb = vt + l16 * kVtStride + g * 16;
#pragma unroll
    for (int et = 0; et < kVDim / 16; ++et) {
      const uint4 av = *reinterpret_cast<const uint4*>(vb + et * 16 * kVtStride);
      o[et] *= alpha;
      o[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), as_bf16x8(pf), o[et], 0, 0, 0);
    }
  }

  // o[et][e] = unnormalised output of head h at dim 16 et + 4 g + e
  const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
  const float lse_v = lsum > 0.f ? m * kLn2 + logf(lsum) : -INFINITY;
  if (p.n_split == 1) {
    uint16_t* orow = static_cast<uint16_t*>(p.out) + ((int64_t)i * p.H + h) * kVDim + 4 * g;
#pragma unroll
    for (int et = 0; et < kVDim / 16; ++et) {
      uint2 v;
      v.x = pack_bf16x2(o[et][0] * inv, o[et][1] * inv);
      v.y = pack_bf16x2(o[et][2] * inv, o[et][3] * inv);
      *reinterpret_cast<uint2*>(orow + et * 16) = v;
    }
    if (p.lse && g == 0) p.lse[(int64_t)i * p.H + h] = lse_v;
  } else {
    float* prow = p.part_o + (((int64_t)split * p.T + i) * p.H + h) * kVDim + 4 * g;
#pragma unroll
    for (int et = 0; et < kVDim / 16; ++et)
      *reinterpret_cast<f32x4*>(prow + et * 16) = o[et] * inv;
    if (g == 0) p.part_lse[((int64_t)split * p.T + i) * p.H + h] = lse_v;
  }
}

// Merge split partials: out = sum_s exp(lse_s - M) o_s / sum_s exp(lse_s - M).
// One 64-lane workgroup per (query row, head), 8 dims per lane; the split
// loop keeps four splits' loads in flight.
template <bool BF16>
__global__ __launch_bounds__(64) void sfa_combine(SfaParams p) {
  const int64_t th = blockIdx.x;  // = i * H + h
  const int lane = threadIdx.x;
  const int64_t stride = (int64_t)p.T * p.H;
  float M = -INFINITY;
  for (int s = 0; s < p.n_split; ++s) M = fmaxf(M, p.part_lse[s * stride + th]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    const float* po = p.part_o + th * kVDim + lane * 8;
    for (int s0 = 0; s0 < p.n_split; s0 += 4) {
      float wgt[4];
      float4 a[4], c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int s = s0 + j;
        const float l = s < p.n_split ? p.part_lse[s * stride + th] : -INFINITY;
        wgt[j] = l == -INFINITY ? 0.f : expf(l - M);
        if (s < p.n_split) {
          a[j] = reinterpret_cast<const float4*>(po + s * stride * kVDim)[0];
          c[j] = reinterpret_cast<const float4*>(po + s * stride * kVDim)[1];
        } else {
          a[j] = c[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        den += wgt[j];
        acc[0] += wgt[j] * a[j].x; acc[1] += wgt[j] * a[j].y; acc[2] += wgt[j] * a[j].z; acc[3] += wgt[j] * a[j].w;
        acc[4] += wgt[j] * c[j].x; acc[5] += wgt[j] * c[j].y; acc[6] += wgt[j] * c[j].z; acc[7] += wgt[j] * c[j].w;
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  if (BF16) {
    uint4 v;
    v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    v.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
    v.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.out) + th * kVDim + lane * 8) = v;
  } else {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.out) + th * kVDim + lane * 8);
    dst[0] = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    dst[1] = make_float4(acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv);
  }
  if (p.lse && lane == 0) p.lse[th] = den > 0.f ? M + logf(den) : -INFINITY;
}

// fp32: one workgroup per (query row, head); logits of all selected rows in
// LDS, then the softmax-weighted sum with each thread owning two output dims.
constexpr int kF32Threads = 256;
constexpr int kF32MaxK = 4096;

__global__ __launch_bounds__(kF32Threads) void sfa_f32(SfaParams p) {
  __shared__ float qsh[kQkDim];
  __shared__ float z[kF32MaxK];
  __shared__ int rowoff[kF32MaxK];  // element offset of each selected row, -1 = none
  __shared__ float red[kF32Threads / 64];
  const int h = blockIdx.x, i = blockIdx.y;
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* q = static_cast<const float*>(p.q) + ((int64_t)i * p.H + h) * kQkDim;
  const float* kv = static_cast<const float*>(p.kv);
  for (int d = tid; d < kQkDim; d += kF32Threads) qsh[d] = q[d];
  const int32_t* irow = p.idx + (int64_t)i * p.K;
  const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
  __syncthreads();
  float lmax = -INFINITY;
  for (int r = tid; r < p.K; r += kF32Threads) {
    const int t = irow[r];
    if (t < 0) {
      rowoff[r] = -1;
      z[r] = -INFINITY;
      continue;
    }
    const int64_t off = ((int64_t)btrow[t >> 6] * kPage + (t & 63)) * kQkDim;
    rowoff[r] = (int)(off / kQkDim);  // row number in the pool
    const float4* row = reinterpret_cast<const float4*>(kv + off);
    float dot = 0.f;
    for (int d = 0; d < kQkDim / 4; ++d) {
      float4 a = row[d];
      dot = fmaf(qsh[4 * d], a.x, dot);
      dot = fmaf(qsh[4 * d + 1], a.y, dot);
      dot = fmaf(qsh[4 * d + 2], a.z, dot);
      dot = fmaf(qsh[4 * d + 3], a.w, dot);
    }
    z[r] = dot * p.scale;
    lmax = fmaxf(lmax, z[r]);
  }
  for (int off = 32; off > 0; off >>= 1) lmax = fmaxf(lmax, __shfl_xor(lmax, off));
  if (lane == 0) red[wave] = lmax;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < kF32Threads / 64; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  float lsum = 0.f;
  if (M != -INFINITY)
    for (int r = tid; r < p.K; r += kF32Threads) {
      const float e = rowoff[r] >= 0 ? expf(z[r] - M) : 0.f;
      z[r] = e;
      lsum += e;
    }
  for (int off = 32; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off);
  if (lane == 0) red[wave] = lsum;
  __syncthreads();
  float L = 0.f;
  for (int w = 0; w < kF32Threads / 64; ++w) L += red[w];
  float acc0 = 0.f, acc1 = 0.f;
  if (M != -INFINITY)
    for (int r = 0; r < p.K; ++r) {
      const int ro = rowoff[r];
      if (ro < 0) continue;
      const float pr = z[r];
      const float* row = kv + (int64_t)ro * kQkDim;
      acc0 = fmaf(pr, row[tid], acc0);
      acc1 = fmaf(pr, row[tid + kF32Threads], acc1);
    }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* out = static_cast<float*>(p.out) + ((int64_t)i * p.H + h) * kVDim;
  out[tid] = acc0 * inv;
  out[tid + kF32Threads] = acc1 * inv;
  if (p.lse && tid == 0) p.lse[(int64_t)i * p.H + h] = L > 0.f ? M + logf(L) : -INFINITY;
}

}  // namespace dsa

using namespace dsa;

template <int NW>
static hipError_t launch_sfa(dim3 grid, size_t lds, hipStream_t s, const SfaParams& p) {
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(sfa_bf16<NW>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sfa_bf16<NW>, grid, dim3(NW * 64), lds, s, p);
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
    hipLaunchKernelGGL(sfa_f32, dim3(a.n_heads, a.num_rows), dim3(kF32Threads), 0, s, p);
    return hipGetLastError();
  }
  // waves per workgroup: 16 heads each, up to 4, dividing the head count
  int nw = 1;
  for (int c = 4; c > 1; --c)
    if ((a.n_heads / 16) % c == 0) { nw = c; break; }
  dim3 grid(a.n_split, a.n_heads / (16 * nw), a.num_rows);
  hipError_t e0;
  const size_t lds = (size_t)kKrowBytes + kVtBytes +
                     (size_t)(a.rows_per_split + kSfaRows - 1) / kSfaRows * kSfaRows * 4;
  switch (nw) {
    case 1: e0 = launch_sfa<1>(grid, lds, s, p); break;
    case 2: e0 = launch_sfa<2>(grid, lds, s, p); break;
    case 3: e0 = launch_sfa<3>(grid, lds, s, p); break;
    default: e0 = launch_sfa<4>(grid, lds, s, p); break;
  }
  if (e0 != hipSuccess) return e0;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  hipLaunchKernelGGL(sfa_combine<true>, dim3(a.num_rows * a.n_heads), dim3(64), 0, s, p);
  return hipGetLastError();
}
