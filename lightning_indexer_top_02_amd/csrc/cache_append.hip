// cache_append.hip -- writes new indexer keys into the paged K pool (gfx950).
//
// The step just before the indexer ("Optimizing Inference for Hybrid
// Attention Architectures: From Operator Fusion to Sequence Sharding",
// section "Breaking Down the Computational Path of Hybrid Attention": each
// new token's normalised key goes to the indexer's K cache, quantized where
// the indexer runs in low precision; section "Layered Quantization:
// Distinguishing Precision Sensitivity" for the MXFP8 grouping).  Key j of
// request b lands at position L_b - n_b + j, where the scoring kernels read
// it.
//
// One group of D/4 consecutive threads per key, four elements per thread:
// the key is read with one 16-byte (fp32) or 8-byte (bf16) load per thread
// and written with one store per thread, so a key's row goes out as whole
// contiguous lines.  The per-token fp8 amax is a reduction over the group's
// lanes, the MXFP8 block amax one over 8 lanes (32 elements).  Pure data
// movement: the kernel is bound by HBM (or, for a decode batch of a few
// keys, by launch latency).
#include "dsa_device.h"

namespace dsa {
namespace {

constexpr int kAppendThreads = 256;

struct AppendParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* bt;
  int bt_stride, max_ctx, num_pages;
  const void* src;
  void* k;
  void* ks;
};

// e4m3 code of x: nearest value with ties to even, saturating at +-448 (the
// largest finite e4m3 value; 0x7F is NaN), sign kept on zero.  Written on
// the fp32 bit pattern: below 2^-6 the codes are the multiples of 2^-9
// (subnormals, the first normal 2^-6 being code 8); above, the 23-bit
// fraction is rounded to 3 bits (the carry may step the exponent) and the
// exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const float a = fabsf(x);
  if (!(a < 448.f)) return sign | 0x7Eu;
  if (a < 0.015625f) return sign | static_cast<uint32_t>(__builtin_rintf(a * 512.f));
  const uint32_t ua = __float_as_uint(a);
  const uint32_t r = (ua + 0x7FFFFu + ((ua >> 20) & 1u)) >> 20;  // (fp32 exponent << 3) | 3 fraction bits
  return sign | (r - (120u << 3));
}

__device__ __forceinline__ uint32_t pack_codes(const float (&v)[4]) {
  return e4m3_code(v[0]) | (e4m3_code(v[1]) << 8) | (e4m3_code(v[2]) << 16) | (e4m3_code(v[3]) << 24);
}

// Maximum over the W lanes of this lane's aligned group of W.
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, W));
  return v;
}

// SRC / DST: 0 fp32, 1 bf16, 2 fp8 (per-token scale), 3 MXFP8.
template <int SRC, int DST, int D>
__global__ __launch_bounds__(kAppendThreads) void li_cache_append(AppendParams p) {
  constexpr int TPT = D / 4;                    // threads per key
  constexpr int KPB = kAppendThreads / TPT;     // keys per workgroup
  const int b = blockIdx.y;
  const int q0 = p.q_offsets[b], nb = p.q_offsets[b + 1] - q0;
  const int part = threadIdx.x % TPT;
  const int j = blockIdx.x * KPB + threadIdx.x / TPT;
  // every check below is uniform over a key's group, so a group runs its
  // lane exchanges with all its lanes or not at all
  if (j >= nb) return;
  const int pos = p.ctx_lens[b] - nb + j;
  if (pos < 0 || pos >= p.max_ctx) return;
  const int phys = p.bt[(int64_t)b * p.bt_stride + pos / kPage];
  if (phys < 0 || phys >= p.num_pages) return;
  const int64_t row = (int64_t)phys * kPage + (pos & (kPage - 1));
  const int64_t e0 = (int64_t)(q0 + j) * D + part * 4;  // first source element of this thread

  float v[4];
  if constexpr (SRC == 0) {
    const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(p.src) + e0);
    v[0] = x.x, v[1] = x.y, v[2] = x.z, v[3] = x.w;
  } else {
    const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.src) + e0);
    v[0] = __uint_as_float(x.x << 16), v[1] = __uint_as_float(x.x & 0xFFFF0000u);
    v[2] = __uint_as_float(x.y << 16), v[3] = __uint_as_float(x.y & 0xFFFF0000u);
  }
  const int64_t o = row * D + part * 4;  // first destination element
  if constexpr (DST == 0) {
    *reinterpret_cast<float4*>(static_cast<float*>(p.k) + o) = make_float4(v[0], v[1], v[2], v[3]);
  } else if constexpr (DST == 1) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    // v_cvt_pk_bf16_f32: round to nearest even
    const uint32_t lo = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{v[0], v[1]}), bf16x2_t));
    const uint32_t hi = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{v[2], v[3]}), bf16x2_t));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.k) + o) = make_uint2(lo, hi);
  } else if constexpr (DST == 2) {
    const float amax = group_max<TPT>(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    const float scale = amax > 0.f ? amax / 448.f : 1.f;  // correctly rounded fp32 division
    float qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = v[i] / scale;
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p.k) + o) = pack_codes(qv);
    if (part == 0) static_cast<float*>(p.ks)[row] = scale;
  } else {
    const float amax = group_max<8>(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
    int e = 0;
    if (amax > 0.f) {
      int ex;
      frexpf(amax, &ex);  // amax = f * 2^ex, f in [0.5, 1): floor(log2 amax) = ex - 1
      e = min(max(ex - 1 - 8, -127), 127);  // minus e4m3's largest exponent
    }
    float qv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) qv[i] = ldexpf(v[i], -e);  // exact
    *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p.k) + o) = pack_codes(qv);
    if ((part & 7) == 0) static_cast<uint8_t*>(p.ks)[row * (D / 32) + part / 8] = static_cast<uint8_t>(e + 127);
  }
}

template <int SRC, int DST, int D>
hipError_t launch(const AppendParams& p, int batch, int max_q, hipStream_t s) {
  constexpr int KPB = kAppendThreads / (D / 4);
  const dim3 grid((max_q + KPB - 1) / KPB, batch);
  hipLaunchKernelGGL((li_cache_append<SRC, DST, D>), grid, dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

template <int SRC, int D>
hipError_t launch_dst(const AppendParams& p, int dst, int batch, int max_q, hipStream_t s) {
  switch (dst) {
    case 0: return launch<SRC, 0, D>(p, batch, max_q, s);
    case 1: return launch<SRC, 1, D>(p, batch, max_q, s);
    case 2: return launch<SRC, 2, D>(p, batch, max_q, s);
    default: return launch<SRC, 3, 128>(p, batch, max_q, s);  // MXFP8: 128-dim only
  }
}

// ---------------------------------------------------------------------------
// Latent rows: each new token's row of the main attention cache (512 latent
// dims, then 64 rope dims), written where sparse attention gathers it.  One
// wave per row: lane l holds latent dims 8l .. 8l + 7 and rope dim l, so each
// lane group of 16 covers one 128-element tile of the fp8 latent row.
// DST 2 is the fp8 latent row ("Day0 Inference Optimization for
// Next-Generation Hybrid-Architecture LLMs Based on CANN", section 3.2: FP8
// per token and 128-element tile): per tile, the exponent e is the smallest
// integer with amax <= 448 * 2^e (0 for a zero tile, at least -126), stored
// as the E8M0 byte e + 127 in a 16-byte block after the codes (the other 12
// bytes zero); codes are the e4m3 codes of x * 2^-e (exact); the rope dims
// follow in bf16.
// ---------------------------------------------------------------------------
constexpr int kLatentRowsPerBlock = kAppendThreads / 64;
constexpr int kF8LatentRow = kVDim + 16 + 2 * (kQkDim - kVDim);  // 656 bytes

struct LatentParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* bt;
  int bt_stride, max_ctx, num_pages;
  const void* src;
  void* kv;
};

__device__ __forceinline__ uint32_t bf16_pack2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{lo, hi}), bf16x2_t));
}

// Smallest e with a <= 448 * 2^e for a > 0 (448 = 1.75 * 2^8): with a =
// m * 2^E, m in [1, 2), that is E - 8, plus one when m > 1.75.  Subnormal a
// (below 2^-126) and anything under the floor give -126.
__device__ __forceinline__ int latent_tile_exponent(float a) {
  if (a == 0.f) return 0;
  const uint32_t u = __float_as_uint(a);
  const int E = (int)(u >> 23) - 127;
  if (E == -127) return -126;
  return max(E - 8 + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0), -126);
}

template <int SRC, int DST>
__global__ __launch_bounds__(kAppendThreads) void li_latent_append(LatentParams p) {
  const int b = blockIdx.y;
  const int q0 = p.q_offsets[b], nb = p.q_offsets[b + 1] - q0;
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * kLatentRowsPerBlock + (threadIdx.x >> 6);
  // uniform over the wave: a row's lanes exchange values only if all go on
  if (j >= nb) return;
  const int pos = p.ctx_lens[b] - nb + j;
  if (pos < 0 || pos >= p.max_ctx) return;
  const int phys = p.bt[(int64_t)b * p.bt_stride + pos / kPage];
  if (phys < 0 || phys >= p.num_pages) return;
  const int64_t row = (int64_t)phys * kPage + (pos & (kPage - 1));
  const int64_t s0 = (int64_t)(q0 + j) * kQkDim;  // first source element of the row

  float v[8], rope;
  if constexpr (SRC == 0) {
    const float* src = static_cast<const float*>(p.src) + s0;
    const float4 x0 = *reinterpret_cast<const float4*>(src + 8 * lane);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 8 * lane + 4);
    v[0] = x0.x, v[1] = x0.y, v[2] = x0.z, v[3] = x0.w, v[4] = x1.x, v[5] = x1.y, v[6] = x1.z, v[7] = x1.w;
    rope = src[kVDim + lane];
  } else {
    const uint16_t* src = static_cast<const uint16_t*>(p.src) + s0;
    const uint4 x = *reinterpret_cast<const uint4*>(src + 8 * lane);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = __uint_as_float(w[k] << 16);
      v[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
    rope = __uint_as_float(static_cast<uint32_t>(src[kVDim + lane]) << 16);
  }
  if constexpr (DST == 0) {
    float* dst = static_cast<float*>(p.kv) + row * kQkDim;
    *reinterpret_cast<float4*>(dst + 8 * lane) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(dst + 8 * lane + 4) = make_float4(v[4], v[5], v[6], v[7]);
    dst[kVDim + lane] = rope;
  } else if constexpr (DST == 1) {
    uint16_t* dst = static_cast<uint16_t*>(p.kv) + row * kQkDim;
    *reinterpret_cast<uint4*>(dst + 8 * lane) =
        make_uint4(bf16_pack2(v[0], v[1]), bf16_pack2(v[2], v[3]), bf16_pack2(v[4], v[5]), bf16_pack2(v[6], v[7]));
    dst[kVDim + lane] = static_cast<uint16_t>(bf16_pack2(rope, 0.f));
  } else {
    uint8_t* dst = static_cast<uint8_t*>(p.kv) + row * kF8LatentRow;
    float amax = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
    const int e = latent_tile_exponent(group_max<16>(amax));  // this lane's tile: dims 128 (lane / 16) ..
    float lo[4], hi[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo[k] = ldexpf(v[k], -e);  // exact
      hi[k] = ldexpf(v[4 + k], -e);
    }
    *reinterpret_cast<uint2*>(dst + 8 * lane) = make_uint2(pack_codes(lo), pack_codes(hi));
    const uint32_t eb = static_cast<uint32_t>(e + 127);
    const uint32_t ew = __shfl(eb, 0) | (__shfl(eb, 16) << 8) | (__shfl(eb, 32) << 16) | (__shfl(eb, 48) << 24);
    if (lane == 0) *reinterpret_cast<uint4*>(dst + kVDim) = make_uint4(ew, 0u, 0u, 0u);
    reinterpret_cast<uint16_t*>(dst + kVDim + 16)[lane] = static_cast<uint16_t>(bf16_pack2(rope, 0.f));
  }
}

template <int SRC, int DST>
hipError_t launch_latent(const LatentParams& p, int batch, int max_q, hipStream_t s) {
  const dim3 grid((max_q + kLatentRowsPerBlock - 1) / kLatentRowsPerBlock, batch);
  hipLaunchKernelGGL((li_latent_append<SRC, DST>), grid, dim3(kAppendThreads), 0, s, p);
  return hipGetLastError();
}

template <int SRC>
hipError_t launch_latent_dst(const LatentParams& p, int dst, int batch, int max_q, hipStream_t s) {
  switch (dst) {
    case 0: return launch_latent<SRC, 0>(p, batch, max_q, s);
    case 1: return launch_latent<SRC, 1>(p, batch, max_q, s);
    default: return launch_latent<SRC, 2>(p, batch, max_q, s);
  }
}

}  // namespace
}  // namespace dsa

using namespace dsa;

hipError_t dsa_launch_latent_append(const DsaLatentAppendLaunch& a, hipStream_t s) {
  if (a.src_dtype < 0 || a.src_dtype > 1 || a.dst_dtype < 0 || a.dst_dtype > 2) return hipErrorInvalidValue;
  if (a.batch < 1 || a.max_q_per_req < 1) return hipSuccess;
  LatentParams p;
  p.q_offsets = a.q_offsets;
  p.ctx_lens = a.ctx_lens;
  p.bt = a.block_table;
  p.bt_stride = a.bt_stride;
  p.max_ctx = a.max_ctx_len;
  p.num_pages = a.num_pages;
  p.src = a.x_new;
  p.kv = a.kv_cache;
  return a.src_dtype == 0 ? launch_latent_dst<0>(p, a.dst_dtype, a.batch, a.max_q_per_req, s)
                          : launch_latent_dst<1>(p, a.dst_dtype, a.batch, a.max_q_per_req, s);
}

hipError_t dsa_launch_cache_append(const DsaAppendLaunch& a, hipStream_t s) {
  if (a.head_dim != 64 && a.head_dim != 128) return hipErrorInvalidValue;
  if (a.dst_dtype == 3 && a.head_dim != 128) return hipErrorInvalidValue;
  if (a.batch < 1 || a.max_q_per_req < 1) return hipSuccess;
  AppendParams p;
  p.q_offsets = a.q_offsets;
  p.ctx_lens = a.ctx_lens;
  p.bt = a.block_table;
  p.bt_stride = a.bt_stride;
  p.max_ctx = a.max_ctx_len;
  p.num_pages = a.num_pages;
  p.src = a.k_new;
  p.k = a.k_cache;
  p.ks = a.k_scale;
  const bool d64 = a.head_dim == 64;
  if (a.src_dtype == 0)
    return d64 ? launch_dst<0, 64>(p, a.dst_dtype, a.batch, a.max_q_per_req, s)
               : launch_dst<0, 128>(p, a.dst_dtype, a.batch, a.max_q_per_req, s);
  return d64 ? launch_dst<1, 64>(p, a.dst_dtype, a.batch, a.max_q_per_req, s)
             : launch_dst<1, 128>(p, a.dst_dtype, a.batch, a.max_q_per_req, s);
}
