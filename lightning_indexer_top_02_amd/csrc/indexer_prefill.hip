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
// A workgroup owns 8 query rows of one request, one per wave.  A wave keeps
// its row's whole query (64 heads x D) in registers as the MFMA A operand and
// walks the request's positions in tiles of 128, which the eight waves share
// through two LDS buffers: while tile t is used, tile t + 1 is written into
// the other buffer (right after the tile's barrier, one barrier per tile),
// tile t + 2's keys are in flight in registers and their block-table entries
// one tile further ahead.
//
// Within a tile a wave takes 32 positions at a time: 64 heads x 32 positions
// x D as MFMAs (one 16x16x128 step for 128-dim fp8, else 16x16x32 steps)
// into 4 x 2 accumulator tiles, with the key fragments
// of each contraction step read from LDS one step ahead.  The epilogue of a
// sub-tile (ReLU, weights, the 64-head sum) is issued together with the
// MFMAs of the next one, on a second accumulator set, so the vector ALU work
// overlaps the matrix cores instead of following them; a tile's four score
// stores follow the tile.  In the
// accumulators the heads of a position sit in one lane column: lane group g
// (lanes 16g .. 16g + 15) holds heads 16t + 4g + i, summed in-lane in
// ascending head order; the four group sums are combined as
// (s0 + s1) + (s2 + s3) with two row permutes, the order of the other indexer
// kernels, so every scoring route gives bit-identical scores.  Tiles past the
// causal edge of a row are skipped.  Each row's level-1 digit histogram (top
// 11 key bits) is complete inside the workgroup, so it is stored without
// atomics for the selection kernel.
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
  const void* q_scale;
  const float* w;
  const void* k;
  const void* k_scale;
  float* scores;
  int64_t score_stride;
  uint32_t* hist;  // [rows][kHistStride]: level-1 histogram at offset 0 (null: scores only)
};

constexpr int kPfThreads = 512;
constexpr int kPfRows = kPfThreads / 64;  // query rows per workgroup
constexpr int kPfTile = 128;              // positions per LDS tile
constexpr int kPfSub = 32;                // positions per MFMA sub-tile
constexpr int kPfHeads = 64;              // heads held in registers (H is padded to this)

template <int DT, int D>
__global__ __launch_bounds__(kPfThreads, 1) void li_prefill(PrefillParams p) {
  using Gm = IdxGeom<DT, D>;
  using frag_t = typename Gm::frag_t;
  constexpr int ES = Gm::ES;
  constexpr int KS = Gm::KS;                     // contraction steps
  constexpr int MT = kPfHeads / 16;              // head tiles
  constexpr int NSUB = kPfTile / kPfSub;         // sub-tiles per tile
  constexpr int KROW = D * ES + 16;              // padded LDS bytes per key row
  constexpr int TILE_BYTES = kPfTile * D * ES;   // key bytes per tile
  constexpr int VPT = TILE_BYTES / 16 / kPfThreads;  // 16-byte loads per thread per tile
  static_assert(NSUB % 2 == 0, "sub-tiles alternate between two accumulator sets");
  extern __shared__ __align__(16) unsigned char smem[];
  // two key tiles: tile t is read from buffer t % 2 while tile t + 1 is
  // written into the other
  unsigned char* const kbuf = smem;                                         // [2][kPfTile][KROW]
  // [2][kPfTile] key scales: fp8 one fp32, MXFP8 the four E8M0 bytes of the position
  float* const kscb = reinterpret_cast<float*>(smem + 2 * kPfTile * KROW);
  uint32_t* lhist = reinterpret_cast<uint32_t*>(kscb + 2 * kPfTile);        // [kPfRows][kHistBins]
  const unsigned char* ktile = kbuf;                                        // the tile being read
  const float* ksc = kscb;

  const int b = blockIdx.y;
  const int q0 = p.q_offsets[b], nb = p.q_offsets[b + 1] - q0;
  // Causal rows: a row block's work grows with its position in the request
  // (row j sees L - n + j + 1 positions), up to twice the average in a
  // prefill from scratch.  Blocks are dispatched heaviest first, so the light
  // ones fill the compute units that the heavy ones leave free at the end
  // instead of the heavy ones running alone in a tail.
  const int r0 = (gridDim.x - 1 - blockIdx.x) * kPfRows;
  if (r0 >= nb) return;
  const int nrows = min(kPfRows, nb - r0);
  const int first_pos = p.ctx_lens[b] - nb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, l16 = lane & 15;
  const bool row_ok = wave < nrows;
  const int row = q0 + r0 + wave;                 // this wave's query row
  const int vis_last = first_pos + r0 + nrows;    // positions any row here sees
  // positions this wave's row sees (wave-uniform: the causal skip below is a
  // scalar branch, not a divergent one)
  const int myvis = __builtin_amdgcn_readfirstlane(row_ok ? first_pos + r0 + wave + 1 : 0);

  for (int c = tid; c < kPfRows * kHistBins; c += kPfThreads) lhist[c] = 0u;

  // this wave's query row as A fragments: qf[mt][ks] = step ks of q[row][mt*16 + l16] for lane group g
  frag_t qf[MT][KS];
  float wl[MT][4];  // weights of heads mt*16 + 4g + i (times the q scale for fp8)
  int qsx[MT];      // MXFP8: the E8M0 scale of block g of head mt*16 + l16 (low byte)
  {
    const unsigned char* qg = static_cast<const unsigned char*>(p.q);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int h = mt * 16 + l16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        frag_t v{};
        if (row_ok && h < p.H)
          v = Gm::load_frag(qg + ((int64_t)row * p.H + h) * (D * ES), ks, g);
        qf[mt][ks] = v;
      }
      qsx[mt] = 0;
      if (Gm::MX && row_ok && h < p.H)
        qsx[mt] = static_cast<const uint8_t*>(p.q_scale)[((int64_t)row * p.H + h) * (D / 32) + g];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int hh = mt * 16 + 4 * g + i;
        float wv = 0.f;
        if (row_ok && hh < p.H) {
          wv = p.w[(int64_t)row * p.H + hh];
          if (DT == 2) wv *= static_cast<const float*>(p.q_scale)[(int64_t)row * p.H + hh];
        }
        wl[mt][i] = wv;
      }
    }
  }

  const int ntiles = (vis_last + kPfTile - 1) / kPfTile;
  const int32_t* btrow = p.bt + (int64_t)b * p.bt_stride;
  const unsigned char* kg = static_cast<const unsigned char*>(p.k);
  constexpr int PPR = D * ES / 16;       // 16-byte pieces per key row
  constexpr int PAGES = kPfTile / kPage;  // pages per tile
  // Block-table entries of a tile's pages, read one tile ahead of the keys so
  // that the key loads never wait on them.  Pages past the last one any row
  // here sees read the last page's entry (every read is issued) and are
  // zero-filled by fetch.
  const int last_pg = (vis_last - 1) / kPage;
  // (read through the constant address space: scalar loads, which leave the
  // vector memory counter to the key loads and score stores)
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr btc = (const_i32_ptr)btrow;
  auto load_phys = [&](int tile, int (&ph)[PAGES]) {
#pragma unroll
    for (int i = 0; i < PAGES; ++i) ph[i] = btc[min(tile * PAGES + i, last_pg)];
  };
  // Every vector memory operation of the tile loop is issued unconditionally
  // (gfx950 counts loads and stores on one in-order counter, and a
  // conditional one makes each wait for a tile's keys a wait for every
  // outstanding store): keys and scales are buffer loads from a resource over
  // one page, and a page past the rows' last position gets an offset beyond
  // the resource, which reads zeros without touching memory.
  constexpr uint32_t kPageBytes = kPage * D * ES;
  constexpr uint32_t kOff = 0x80000000u;  // out of every resource's range
  uint4 pre[VPT];
  float pre_s = 0.f;
  // the keys of tile `tile`, whose block-table entries are ph
  auto fetch = [&](int tile, const int (&ph_raw)[PAGES]) {
    int ph[PAGES];
#pragma unroll
    for (int i = 0; i < PAGES; ++i) ph[i] = tile * PAGES + i <= last_pg ? ph_raw[i] : -1;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int c = tid + j * kPfThreads;  // 16-byte piece of the tile
      const int pos = c / PPR;             // position within the tile
      const int part = c - pos * PPR;
      int phys = ph[0];
#pragma unroll
      for (int i = 1; i < PAGES; ++i) phys = (pos >> 6) == i ? ph[i] : phys;
      // a wave's 1 KB of pieces lies in one page, so phys is wave-uniform
      phys = __builtin_amdgcn_readfirstlane(phys);
      const auto rs = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<unsigned char*>(kg) + (phys >= 0 ? (int64_t)phys * kPageBytes : 0), 0, kPageBytes, 0x00020000);
      const uint32_t off = phys >= 0 ? (uint32_t)((pos & 63) * (D * ES) + part * 16) : kOff;
      pre[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
    }
    if constexpr (DT >= 2) {
      // threads below kPfTile load the scale of tile position tid (fp8: one
      // fp32, MXFP8: the four E8M0 bytes of the position)
      int phys = ph[0];
#pragma unroll
      for (int i = 1; i < PAGES; ++i) phys = (tid >> 6) == i ? ph[i] : phys;
      phys = __builtin_amdgcn_readfirstlane(phys);
      const auto rsc = __builtin_amdgcn_make_buffer_rsrc(
          static_cast<unsigned char*>(const_cast<void*>(p.k_scale)) + (phys >= 0 ? (int64_t)phys * kPage * 4 : 0), 0,
          kPage * 4, 0x00020000);
      const uint32_t off = (phys >= 0 && tid < kPfTile) ? (uint32_t)(tid & 63) * 4u : kOff;
      pre_s = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsc, (int)off, 0, 0));
    }
  };
  auto stage = [&](int buf) {
    unsigned char* kt = kbuf + buf * kPfTile * KROW;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int c = tid + j * kPfThreads;
      const int pos = c / PPR;
      const int part = c - pos * PPR;
      *reinterpret_cast<uint4*>(kt + pos * KROW + part * 16) = pre[j];
    }
    if (DT >= 2 && tid < kPfTile) kscb[buf * kPfTile + tid] = pre_s;
  };

  // Two accumulator sets: the MFMAs of a sub-tile go to one while the
  // epilogue of the previous sub-tile reads the other.
  f32x4 acc[2][MT][2];
  float sc_k[2] = {1.f, 1.f};  // fp8: this lane's key scale, per set
  // B fragments of contraction step ks of sub-tile sub (positions sub*32 + pt*16 + l16)
  auto load_b = [&](frag_t (&bf)[2], int sub, int ks) {
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
      bf[pt] = Gm::load_frag(ktile + (sub * kPfSub + pt * 16 + l16) * KROW, ks, g);
  };
  // The MFMAs of one sub-tile.  bf holds its first step's fragments on entry;
  // every step loads the next step's fragments (the next sub-tile's first one
  // at the end, when there is one in this tile) before its own MFMAs, so the
  // LDS latency is hidden behind them.
  auto mfma_sub = [&](f32x4 (&a)[MT][2], float& kscale, int sub, frag_t (&bf)[2]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) a[mt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
    int kx[2] = {0, 0};  // MXFP8: block g scale of position sub*32 + pt*16 + l16 (low byte)
    if constexpr (Gm::MX) {
#pragma unroll
      for (int pt = 0; pt < 2; ++pt) kx[pt] = (int)(__float_as_uint(ksc[sub * kPfSub + pt * 16 + l16]) >> (8 * g));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      frag_t cur[2] = {bf[0], bf[1]};
      if (ks + 1 < KS) load_b(bf, sub, ks + 1);
      else if (sub + 1 < NSUB) load_b(bf, sub + 1, 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
          if constexpr (Gm::MX) a[mt][pt] = mfma_step_mx(qf[mt][ks], cur[pt], a[mt][pt], qsx[mt], kx[pt]);
          else a[mt][pt] = mfma_step(qf[mt][ks], cur[pt], a[mt][pt]);
        }
    }
    // the scale of the position this lane ends up holding (lanes g < 2)
    if (DT == 2) kscale = ksc[sub * kPfSub + (g & 1) * 16 + l16];
  };
  // a[mt][pt][i] = logit of head mt*16 + 4g + i at position sub*32 + pt*16 + l16.
  // Returns, on lanes g < 2, the score of position 16 (g & 1) + l16 of the
  // sub-tile: in-lane group sums of each position tile, then two row swaps
  // (VALU permutes, no LDS): lanes 16-row r and r^1 exchange so that even
  // rows add up tile 0 and odd rows tile 1 of groups g, g^1, then the 32-lane
  // halves exchange and add, giving (s0 + s1) + (s2 + s3).
  auto epilogue = [&](const f32x4 (&a)[MT][2], float kscale) {
    float sp[2];
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
      float s = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) s += wl[mt][i] * relu_keep_nan(a[mt][pt][i]);
      sp[pt] = s;
    }
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(sp[0]), __float_as_uint(sp[1]), false, false);
    const float pair = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(pair), __float_as_uint(pair), false, false);
    float s = __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
    if (DT == 2) s *= kscale;
    return s;
  };
  // This wave's score row as a buffer of myvis positions: lanes g < 2 store
  // the score of sub-tile position base + 16 (g & 1) + l16 (base < 0: none);
  // the other lanes, and positions the row does not see, get offsets past the
  // buffer, which the hardware drops.
  const int srow_row = __builtin_amdgcn_readfirstlane(row_ok ? row : 0);  // (wave-uniform)
  const auto srow = __builtin_amdgcn_make_buffer_rsrc(p.scores + (int64_t)srow_row * p.score_stride, 0, myvis * 4,
                                                      0x00020000);
  // (sub: which store of the tile, so that dropped stores get distinct
  // offsets and are not merged into one)
  auto store = [&](float s, int base, int sub) {
    const int pos = base + (g & 1) * 16 + l16;
    const bool on = g < 2 && base >= 0;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(s), srow,
                                          (int)(on ? (uint32_t)pos * 4u : kOff + 4u * (uint32_t)sub), 0, 0);
  };
  auto count = [&](float s, int base) {
    const int pos = base + (g & 1) * 16 + l16;
    if (g < 2 && base >= 0 && pos < myvis) atomicAdd(&lhist[wave * kHistBins + (score_key(s) >> kLevelShift[0])], 1u);
  };

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) acc[1][mt][pt] = f32x4{0.f, 0.f, 0.f, 0.f};
  int pending = -1;  // first position of the sub-tile waiting in acc[1], or -1

  int ph_next[PAGES];
  load_phys(0, ph_next);  // (ntiles >= 1: every workgroup has a row)
  fetch(0, ph_next);
  stage(0);
  load_phys(1, ph_next);
  fetch(1, ph_next);  // (past the last tile: zeros)
  load_phys(2, ph_next);
  // dropped stores in place of a tile's score stores: the memory operations
  // before the loop then end as each pass through it ends, and the counts the
  // compiler derives for the loop's waits hold on the first pass too (else
  // the block-table reads just above make every tile wait for everything)
  __builtin_amdgcn_sched_barrier(0);  // (kept after the reads above)
#pragma unroll
  for (int sub = 0; sub < NSUB; ++sub) store(0.f, -1, sub);
  for (int tile = 0; tile < ntiles; ++tile) {
    __syncthreads();  // tile is staged; the other buffer (tile - 1) is no longer read
    ktile = kbuf + (tile & 1) * kPfTile * KROW;
    ksc = kscb + (tile & 1) * kPfTile;
    // tile + 1 goes into the other buffer (its loads have had a whole tile to
    // arrive), and tile + 2's loads start; past the last tile they are zeros,
    // staged into a buffer nobody reads.  This comes before the causal skip,
    // so both paths hold the tiles in the same registers and issue the same
    // memory operations (else every wait for a tile waits for all stores too).
    stage((tile + 1) & 1);
    fetch(tile + 2, ph_next);
    load_phys(tile + 3, ph_next);
    // A tile's four sub-tile scores are stored after the tile, from one
    // place for the scored and the skipped tiles (whose stores are dropped),
    // so every path through the loop issues the same memory operations in the
    // same order.
    float s_out[NSUB];
    int b_out[NSUB];
    if (tile * kPfTile < myvis) {  // (never for a wave without a row)
      frag_t bf[2];
      load_b(bf, 0, 0);
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        const int cur = sub & 1;
        // the previous sub-tile (the last one of the previous tile when sub == 0)
        b_out[sub] = sub == 0 ? pending : tile * kPfTile + (sub - 1) * kPfSub;
        mfma_sub(acc[cur], sc_k[cur], sub, bf);
        s_out[sub] = epilogue(acc[cur ^ 1], sc_k[cur ^ 1]);
        count(s_out[sub], b_out[sub]);
      }
      pending = tile * kPfTile + (NSUB - 1) * kPfSub;
    } else {
#pragma unroll
      for (int sub = 0; sub < NSUB; ++sub) {
        s_out[sub] = 0.f;
        b_out[sub] = -1;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) store(s_out[sub], b_out[sub], sub);
  }
  {
    const float sl = epilogue(acc[1], sc_k[1]);
    store(sl, pending, 0);
    count(sl, pending);
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
  const size_t lds = 2 * ((size_t)kPfTile * (D * Gm::ES + 16) + kPfTile * 4) + (size_t)kPfRows * kHistBins * 4;
  {
    const hipError_t e = dsa_allow_lds(reinterpret_cast<const void*>(li_prefill<DT, D>), lds);
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
  return a.max_q_per_req > 4 && a.num_rows >= 1024;
}

// Scores and level-1 histograms of every row (bf16, fp8 or MXFP8 keys, at most 64
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
  if (a.dtype == 3) return launch_prefill<3, 128>(p, grid, s);  // MXFP8: 128-dim only
  return d64 ? launch_prefill<2, 64>(p, grid, s) : launch_prefill<2, 128>(p, grid, s);
}
