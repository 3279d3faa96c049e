// indexer_common.h -- lightning-indexer scoring shared by the indexer kernels.
//
// Score of position t for one query row ("Optimizing Inference for Hybrid
// Attention Architectures: From Operator Fusion to Sequence Sharding",
// section "Breaking Down the Computational Path of Hybrid Attention", item 1):
//     s_t = sum_h w_h * max(q_h . k_t, 0)
// fp8 route: q_h . k_t = (q̂_h . k̂_t) * sq_h * sk_t with positive scales, so
// sq_h is folded into w_h and sk_t applied after the head sum.
//
// bf16/fp8 keys use MFMA: logits D[m = head][n = position] with the query
// rows as A (from LDS) and the keys as B, loaded straight from the page in
// HBM.  bf16 and 64-dim fp8 take 16x16x32 steps (each lane reads 8
// consecutive elements of one key row); 128-dim fp8 takes one 16x16x128
// step, gfx950's only fp8 MFMA that runs at twice the bf16 rate (a 16x16x32
// fp8 MFMA takes as long as a bf16 one).  fp32 keys use VALU, one thread per
// position.  MXFP8 (128-dim) takes the same 16x16x128 step in its
// block-scaled form: the fragment layout below feeds element j of a row as
// contraction index j, the instruction scales contraction indices 32b ..
// 32b + 31 by the E8M0 operand of lane group b of that row or column, so
// lane group g passes the scale of its row's block g.
#pragma once

#include <type_traits>

#include "dsa_device.h"

namespace dsa {

// ReLU as one integer max on the bit pattern: a set sign bit reads as a
// negative int32, so every negative value (and -0) becomes +0, while positive
// values, +Inf and NaNs with a clear sign bit (the kind arithmetic on a NaN
// produces) pass unchanged, so a stray read of poisoned cache data still shows
// up in the result.  A compare and select would cost two vector instructions
// per logit, and the ReLU runs once for every (head, position) pair.
__device__ __forceinline__ float relu_keep_nan(float v) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, v), 0));
}

// 32 fp8 elements per lane: the operand of one 16x16x128 step.
struct Frag8 {
  uint4 lo, hi;
};

// One contraction step of a 16x16 tile: D = A B + C.
__device__ __forceinline__ f32x4 mfma_step(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_step(uint2 a, uint2 b, f32x4 c) {
  long la = __builtin_bit_cast(long, a), lb = __builtin_bit_cast(long, b);
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(la, lb, c, 0, 0, 0);
}
// The 16x16x128 step with E8M0 scales: sa for this lane's A block, sb for
// its B block (low bytes).
__device__ __forceinline__ f32x4 mfma_step_mx(const Frag8& a, const Frag8& b, f32x4 c, int sa, int sb) {
  typedef int v8i __attribute__((ext_vector_type(8)));
  const v8i va = {(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w, (int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w};
  const v8i vb = {(int)b.lo.x, (int)b.lo.y, (int)b.lo.z, (int)b.lo.w, (int)b.hi.x, (int)b.hi.y, (int)b.hi.z, (int)b.hi.w};
  // formats 0, 0: both operands fp8 e4m3
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(va, vb, c, 0, 0, 0, sa, 0, sb);
}
__device__ __forceinline__ f32x4 mfma_step(const Frag8& a, const Frag8& b, f32x4 c) {
  // zero scale operands select the unscaled instruction (v_mfma_f32_16x16x128_f8f6f4)
  return mfma_step_mx(a, b, c, 0, 0);
}

// Storage geometry of one indexer variant: DT 0 = fp32, 1 = bf16, 2 = fp8,
// 3 = MXFP8 (128-dim only).
template <int DT, int D>
struct IdxGeom {
  static constexpr int ES = DT == 0 ? 4 : (DT == 1 ? 2 : 1);   // bytes per element
  // LDS bytes per (row, head); MXFP8 keeps the D/32 block scales of the
  // (row, head) in the 16 bytes after its codes
  static constexpr int QSTRIDE = DT == 0 ? D * 4 : D * ES + 16;
  static constexpr bool MX = DT == 3;
  static_assert(!MX || D == 128, "MXFP8 takes one 16x16x128 step");
  static constexpr bool K128 = DT >= 2 && D == 128;             // one 16x16x128 fp8 step
  static constexpr int KS = K128 ? 1 : D / 32;                  // contraction steps
  using frag_t = typename std::conditional<K128, Frag8, typename std::conditional<DT == 1, uint4, uint2>::type>::type;
  // Byte offset, within a row of D elements, of the 8 elements lane group g
  // feeds to the MFMA at contraction step ks.  Any assignment of the row's
  // elements to (ks, g) gives the same dot product as long as the query and
  // key fragments use the same one; bf16 takes elements 32 ks + 8g .. + 8.
  // fp8 pairs the steps so that lane group g reads 16 contiguous bytes at
  // 16g + 64 j (steps 2j and 2j + 1): each load instruction then covers 64
  // contiguous bytes of every key row instead of 32.  The 16x16x128 step
  // takes the same 32 bytes per lane group at once (16g .. and 64 + 16g ..).
  static __host__ __device__ constexpr int frag_byte(int ks, int g) {
    return DT >= 2 ? 16 * g + 8 * (ks & 1) + 64 * (ks >> 1) : (32 * ks + 8 * g) * ES;
  }
  // The fragment of contraction step ks for lane group g of the row at `row`.
  static __device__ __forceinline__ frag_t load_frag(const unsigned char* row, int ks, int g) {
    if constexpr (K128) {
      return Frag8{*reinterpret_cast<const uint4*>(row + 16 * g), *reinterpret_cast<const uint4*>(row + 64 + 16 * g)};
    } else {
      return *reinterpret_cast<const frag_t*>(row + frag_byte(ks, g));
    }
  }
};

// LDS bytes for the staged queries and weights of `rows` rows.
template <int DT, int D>
__host__ __device__ constexpr size_t query_lds_bytes(int rows, int Hpad) {
  return (size_t)rows * Hpad * (IdxGeom<DT, D>::QSTRIDE + 4);
}

// Stage `nrows` query rows starting at global row `row0` (heads past H are
// zero) and their weights (times the q scale for fp8) into LDS; MXFP8 rows
// keep their block scales beside the codes (padded heads: 2^0).
template <int DT, int D, int NT>
__device__ void stage_queries(unsigned char* qs, float* wsm, const void* q, const void* q_scale,
                              const float* w, int row0, int nrows, int H, int Hpad) {
  using G = IdxGeom<DT, D>;
  constexpr int CPH = D * G::ES / 16;  // 16-byte chunks per head
  const unsigned char* qg = static_cast<const unsigned char*>(q);
  const int total = nrows * Hpad * CPH;
  for (int c = threadIdx.x; c < total; c += NT) {
    const int r = c / (Hpad * CPH);
    const int rem = c - r * Hpad * CPH;
    const int h = rem / CPH, part = rem - h * CPH;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (h < H) v = *reinterpret_cast<const uint4*>(qg + ((int64_t)(row0 + r) * H + h) * (D * G::ES) + part * 16);
    *reinterpret_cast<uint4*>(qs + (r * Hpad + h) * G::QSTRIDE + part * 16) = v;
  }
  if constexpr (G::MX) {
    for (int c = threadIdx.x; c < nrows * Hpad; c += NT) {
      const int r = c / Hpad, h = c - r * Hpad;
      const uint32_t e = h < H ? static_cast<const uint32_t*>(q_scale)[(int64_t)(row0 + r) * H + h] : 0x7f7f7f7fu;
      *reinterpret_cast<uint32_t*>(qs + (r * Hpad + h) * G::QSTRIDE + D) = e;
    }
  }
  for (int c = threadIdx.x; c < nrows * Hpad; c += NT) {
    const int r = c / Hpad, h = c - r * Hpad;
    float wv = 0.f;
    if (h < H) {
      const int64_t o = (int64_t)(row0 + r) * H + h;
      wv = w[o];
      if (DT == 2) wv *= static_cast<const float*>(q_scale)[o];  // q scale > 0 folds through the ReLU
    }
    wsm[r * Hpad + h] = wv;
  }
}

// Key fragments of NPT tiles of 16 positions of one page (slots slot0 ..
// slot0 + 16 NPT - 1), in the B-operand layout: kf[pt][ks] holds 8 elements
// of position slot0 + pt*16 + l16 at byte frag_byte(ks, g); kscale[pt] its
// fp8 scale (1 otherwise); kmx[pt] its MXFP8 block-g scale.
template <int DT, int D, int NPT>
struct KeyTiles {
  typename IdxGeom<DT, D>::frag_t kf[NPT][IdxGeom<DT, D>::KS];
  float kscale[NPT];
  int kmx[NPT];
};

// The key scales of physical page `phys` (fp8: one fp32 per slot; MXFP8:
// D/32 E8M0 bytes per slot), or null.
template <int DT, int D>
__device__ __forceinline__ const void* page_scales(const void* k_scale, int64_t phys) {
  if constexpr (DT == 2) return static_cast<const float*>(k_scale) + phys * kPage;
  if constexpr (DT == 3) return static_cast<const uint8_t*>(k_scale) + phys * kPage * (D / 32);
  return nullptr;
}

template <int DT, int D, int NPT>
__device__ __forceinline__ void load_key_tiles(KeyTiles<DT, D, NPT>& t, const unsigned char* kpage,
                                               const void* kscale_page, int slot0) {
  using G = IdxGeom<DT, D>;
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
    for (int ks = 0; ks < G::KS; ++ks)
      t.kf[pt][ks] = G::load_frag(kpage + (uint32_t)(slot0 + pt * 16 + l16) * (uint32_t)(D * G::ES), ks, g);
#pragma unroll
  for (int pt = 0; pt < NPT; ++pt) {
    const int slot = slot0 + pt * 16 + l16;
    t.kscale[pt] = DT == 2 ? static_cast<const float*>(kscale_page)[(uint32_t)slot] : 1.f;
    t.kmx[pt] = DT == 3 ? static_cast<const uint8_t*>(kscale_page)[(uint32_t)(slot * (D / 32) + g)] : 0;
  }
}

// One wave scores NPT loaded key tiles for `nrows` staged rows.  emit(r,
// slot, score) runs on lanes 0..15 for slots slot0 + pt * 16 + lane, except
// on the two unrolled shapes of four values per lane group: with NR = 4
// every lane emits row g (lane group g) for each tile, and with NR = 1 and
// NPT = 4 every lane emits slot slot0 + lane (tile g), so the head sums are
// split over the lane groups by group4_sum_scatter and every emit runs on
// all 64 lanes.  NR > 0 and MT > 0 fix the row count and Hpad / 16 at
// compile time: the row and head-tile loops are then fully unrolled, so no
// loop reads the key registers (a loop that does makes the compiler wait for
// every outstanding vector load before entering it, prefetched tiles
// included).  The sums are formed in the same order on every shape.
template <int DT, int D, int NPT, int NR = 0, int MT = 0, class Emit>
__device__ __forceinline__ void score_key_tiles(const unsigned char* qs, const float* wsm, int Hpad, int nrows,
                                                const KeyTiles<DT, D, NPT>& t, int slot0, Emit&& emit) {
  using G = IdxGeom<DT, D>;
  constexpr int KS = G::KS;  // contraction steps
  const int lane = threadIdx.x & 63, g = lane >> 4, l16 = lane & 15;
  const int hp = MT > 0 ? 16 * MT : Hpad;
  auto head_tile = [&](int r, int ht, float (&sacc)[NPT]) {
    f32x4 acc[NPT];
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) acc[pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const unsigned char* qrow = qs + (r * hp + ht * 16 + l16) * G::QSTRIDE;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const typename G::frag_t a = G::load_frag(qrow, ks, g);
      if constexpr (G::MX) {
        const int sa = qrow[D + g];
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) acc[pt] = mfma_step_mx(a, t.kf[pt][ks], acc[pt], sa, t.kmx[pt]);
      } else {
#pragma unroll
        for (int pt = 0; pt < NPT; ++pt) acc[pt] = mfma_step(a, t.kf[pt][ks], acc[pt]);
      }
    }
    // acc[pt][i] = logit of head ht*16 + 4g + i at slot slot0 + pt*16 + l16
    const float* wr = wsm + r * hp + ht * 16 + 4 * g;
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[pt] += wr[i] * relu_keep_nan(acc[pt][i]);
  };
  // per-lane partial head sums of row r for each tile
  auto row_sums = [&](int r, float (&sacc)[NPT]) {
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) sacc[pt] = 0.f;
    if constexpr (MT > 0) {
#pragma unroll
      for (int ht = 0; ht < MT; ++ht) head_tile(r, ht, sacc);
    } else {
      for (int ht = 0; ht < Hpad / 16; ++ht) head_tile(r, ht, sacc);
    }
  };
  if constexpr (NR == 4) {
    float sacc[4][NPT];
    // rows one after another: each row's sums are pinned (empty asm) before
    // the next row starts, else the compiler defers the epilogues and keeps
    // all four rows' MFMA results, which no longer fit the registers
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      row_sums(r, sacc[r]);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) asm volatile("" : "+v"(sacc[r][pt]));
    }
#pragma unroll
    for (int pt = 0; pt < NPT; ++pt) {
      const float x[4] = {sacc[0][pt], sacc[1][pt], sacc[2][pt], sacc[3][pt]};
      emit(g, slot0 + pt * 16 + l16, group4_sum_scatter(x) * t.kscale[pt]);
    }
  } else if constexpr (NR == 1 && NPT == 4) {
    float sacc[4];
    row_sums(0, sacc);
    const float ks = g == 0 ? t.kscale[0] : (g == 1 ? t.kscale[1] : (g == 2 ? t.kscale[2] : t.kscale[3]));
    emit(0, slot0 + lane, group4_sum_scatter(sacc) * ks);
  } else {
    auto row = [&](int r) {
      float sacc[NPT];
      row_sums(r, sacc);
#pragma unroll
      for (int pt = 0; pt < NPT; ++pt) {
        const float s = group4_sum(sacc[pt]);
        if (g == 0) emit(r, slot0 + pt * 16 + l16, s * t.kscale[pt]);
      }
    };
    if constexpr (NR > 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) row(r);
    } else {
      for (int r = 0; r < nrows; ++r) row(r);
    }
  }
}

// One thread scores one fp32 key row for `nrows` staged rows.
template <int D, class Emit>
__device__ __forceinline__ void score_pos_f32(const float* qs, const float* wsm, int H, int nrows,
                                              const float* krow_ptr, Emit&& emit) {
  const float4* krow = reinterpret_cast<const float4*>(krow_ptr);
  float4 kr[D / 4];
#pragma unroll
  for (int d = 0; d < D / 4; ++d) kr[d] = krow[d];
  for (int r = 0; r < nrows; ++r) {
    float s = 0.f;
    for (int h = 0; h < H; ++h) {
      const float4* qh = reinterpret_cast<const float4*>(qs + (r * H + h) * D);
      float logit = 0.f;
#pragma unroll
      for (int d = 0; d < D / 4; ++d) {
        const float4 qv = qh[d];
        logit = fmaf(qv.x, kr[d].x, logit);
        logit = fmaf(qv.y, kr[d].y, logit);
        logit = fmaf(qv.z, kr[d].z, logit);
        logit = fmaf(qv.w, kr[d].w, logit);
      }
      s = fmaf(wsm[r * H + h], relu_keep_nan(logit), s);
    }
    emit(r, s);
  }
}

}  // namespace dsa
