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
// and one contiguous slice of the row's index list.  The selected rows are
// gathered through the block table in chunks of 32 into LDS (the scattered
// reads become 1152-byte row reads, "aggregating random small reads",
// "Optimizing Inference for Hybrid Attention LLMs: Practices for Fast
// Adaptation", section 3, item 2), and every wave of the workgroup reuses
// them.  Per chunk and wave, MFMA computes S^T = K Q^T (32 rows x 16 heads,
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

template <int NW>
__global__ __launch_bounds__(NW * 64) void sfa_bf16(SfaParams p) {
  __shared__ __align__(16) unsigned char kvs[kSfaRows * kRowStride];
  __shared__ int rvalid[kSfaRows];
  constexpr int NT = NW * 64;
  const int split = blockIdx.x, hg = blockIdx.y, i = blockIdx.z;
  const int b = request_of_row(p.q_offsets, p.batch, i);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const int h = hg * (16 * NW) + wave * 16 + l16;  // this lane's head column

  // Q fragments of this lane's head: qf[s] = q[h][32 s + 8 g .. + 8]
  uint4 qf[kQkDim / 32];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + ((int64_t)i * p.H + h) * kQkDim;
#pragma unroll
    for (int s = 0; s < kQkDim / 32; ++s) qf[s] = *reinterpret_cast<const uint4*>(qrow + s * 32 + g * 8);
  }
  f32x4 o[kVDim / 16];
#pragma unroll
  for (int et = 0; et < kVDim / 16; ++et) o[et] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, lsum = 0.f;
  const float zscale = p.scale * kLog2e;

  const int r_begin = split * p.rows_per_split;
  const int r_end = min(p.K, r_begin + p.rows_per_split);
  const int32_t* irow = p.idx + (int64_t)i * p.K;
  const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
  const uint16_t* kvg = static_cast<const uint16_t*>(p.kv);

  for (int c0 = r_begin; c0 < r_end; c0 += kSfaRows) {
    __syncthreads();
    for (int c = tid; c < kSfaRows * (kRowBytes / 16); c += NT) {
      const int r = c / (kRowBytes / 16), part = c - r * (kRowBytes / 16);
      const int rr = c0 + r;
      const int t = rr < r_end ? irow[rr] : -1;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (t >= 0) {
        const int phys = btrow[t >> 6];
        v = *reinterpret_cast<const uint4*>(kvg + ((int64_t)phys * kPage + (t & 63)) * kQkDim + part * 8);
      }
      *reinterpret_cast<uint4*>(kvs + r * kRowStride + part * 16) = v;
      if (part == 0) rvalid[r] = t >= 0;
    }
    __syncthreads();

    // S^T tiles: s0[i] = S[head l16][row 4g+i], s1[i] = S[head l16][row 16+4g+i]
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* ka = kvs + l16 * kRowStride + g * 16;
#pragma unroll
    for (int s = 0; s < kQkDim / 32; ++s) {
      uint4 a0 = *reinterpret_cast<const uint4*>(ka + s * 64);
      uint4 a1 = *reinterpret_cast<const uint4*>(ka + 16 * kRowStride + s * 64);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a0), as_bf16x8(qf[s]), s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a1), as_bf16x8(qf[s]), s1, 0, 0, 0);
    }
    float z[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[e] = rvalid[4 * g + e] ? s0[e] * zscale : -INFINITY;
      z[4 + e] = rvalid[16 + 4 * g + e] ? s1[e] * zscale : -INFINITY;
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

    // B operand of O^T += V^T P^T: element e of lane group g is row r(e) with
    // r(e) = 4g + e (e < 4) and 16 + 4g + e - 4 (e >= 4), the rows this lane
    // already holds in s0/s1.
    uint4 pf;
    pf.x = pack_bf16x2(pr[0], pr[1]);
    pf.y = pack_bf16x2(pr[2], pr[3]);
    pf.z = pack_bf16x2(pr[4], pr[5]);
    pf.w = pack_bf16x2(pr[6], pr[7]);
    const uint16_t* vb = reinterpret_cast<const uint16_t*>(kvs) + l16;
    const int rs = kRowStride / 2;
#pragma unroll
    for (int et = 0; et < kVDim / 16; ++et) {
      const uint16_t* vc = vb + et * 16;
      uint4 va;
      va.x = (uint32_t)vc[(4 * g + 0) * rs] | ((uint32_t)vc[(4 * g + 1) * rs] << 16);
      va.y = (uint32_t)vc[(4 * g + 2) * rs] | ((uint32_t)vc[(4 * g + 3) * rs] << 16);
      va.z = (uint32_t)vc[(16 + 4 * g + 0) * rs] | ((uint32_t)vc[(16 + 4 * g + 1) * rs] << 16);
      va.w = (uint32_t)vc[(16 + 4 * g + 2) * rs] | ((uint32_t)vc[(16 + 4 * g + 3) * rs] << 16);
      o[et] *= alpha;
      o[et] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va), as_bf16x8(pf), o[et], 0, 0, 0);
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
// One wave per (query row, head), 8 dims per lane.
template <bool BF16>
__global__ __launch_bounds__(256) void sfa_combine(SfaParams p) {
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= p.T * p.H) return;
  const int lane = threadIdx.x & 63;
  const int64_t th = w;  // = i * H + h
  float M = -INFINITY;
  for (int s = 0; s < p.n_split; ++s) M = fmaxf(M, p.part_lse[s * (int64_t)p.T * p.H + th]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
    for (int s = 0; s < p.n_split; ++s) {
      const float l = p.part_lse[s * (int64_t)p.T * p.H + th];
      if (l == -INFINITY) continue;
      const float wgt = expf(l - M);
      den += wgt;
      const float4* src = reinterpret_cast<const float4*>(p.part_o + (s * (int64_t)p.T * p.H + th) * kVDim + lane * 8);
      float4 a = src[0], c = src[1];
      acc[0] += wgt * a.x; acc[1] += wgt * a.y; acc[2] += wgt * a.z; acc[3] += wgt * a.w;
      acc[4] += wgt * c.x; acc[5] += wgt * c.y; acc[6] += wgt * c.z; acc[7] += wgt * c.w;
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
  switch (nw) {
    case 1: hipLaunchKernelGGL(sfa_bf16<1>, grid, dim3(64), 0, s, p); break;
    case 2: hipLaunchKernelGGL(sfa_bf16<2>, grid, dim3(128), 0, s, p); break;
    case 3: hipLaunchKernelGGL(sfa_bf16<3>, grid, dim3(192), 0, s, p); break;
    default: hipLaunchKernelGGL(sfa_bf16<4>, grid, dim3(256), 0, s, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  const int waves = a.num_rows * a.n_heads;
  hipLaunchKernelGGL(sfa_combine<true>, dim3((waves + 3) / 4), dim3(256), 0, s, p);
  return hipGetLastError();
}
