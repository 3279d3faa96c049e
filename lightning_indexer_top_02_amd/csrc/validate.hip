// validate.hip -- device-side check of the paging data the other entry points
// trust (gfx950).
//
// Every kernel of the library translates a position t of request b through
// the block table, page block_table[b][t / 64] and slot t % 64 ("Optimizing
// Inference for Hybrid Attention LLMs: Practices for Fast Adaptation",
// section 3.2; "Day0 Inference Support and Performance Optimization for New
// LLM Architectures", section III, 3.2), and takes the rows of request b from
// q_offsets.  Those arrays live on the device, so the host checks of the
// entry points cannot see them; a page id outside the pool or a context
// longer than the bounds the grids were sized for is undefined behaviour
// there.  This kernel reads them, and only them, and reports what is wrong as
// an OR of flag bits.
//
// One workgroup: thread i checks requests i, i + 1024, ... and then the
// block-table entries of the pages each request uses, read as one flat list
// of (request, page) pairs.  The flags meet in an LDS word, and thread 0
// stores the result with a plain store (no read-modify-write of the output,
// so it needs no clearing first and the launch may be captured in a graph).
#include "dsa_device.h"

namespace dsa {

constexpr int kValidateThreads = 1024;

struct ValidateParams {
  const int32_t* q_offsets;
  const int32_t* ctx_lens;
  const int32_t* block_table;
  int batch, num_q_tokens, max_q_per_req, max_ctx_len, max_pages_per_req, num_pages;
  uint32_t* error_word;
};

__global__ __launch_bounds__(kValidateThreads) void validate_paged(ValidateParams p) {
  __shared__ uint32_t flags;
  const int tid = threadIdx.x;
  if (tid == 0) flags = 0u;
  __syncthreads();
  uint32_t f = 0u;
  if (tid == 0 && (p.q_offsets[0] != 0 || p.q_offsets[p.batch] != p.num_q_tokens)) f |= kValidQOffsets;
  for (int b = tid; b < p.batch; b += kValidateThreads) {
    const int n = p.q_offsets[b + 1] - p.q_offsets[b];
    const int len = p.ctx_lens[b];
    if (n < 0) f |= kValidQOffsets;
    if (n > p.max_q_per_req) f |= kValidRows;
    if (len < n || len > p.max_ctx_len) f |= kValidCtxLen;
    if (len > 0 && (len + kPage - 1) / kPage > p.max_pages_per_req) f |= kValidPageCount;
  }
  // the block-table entries of the pages each request uses (never past its
  // row of max_pages_per_req entries)
  const int64_t pairs = (int64_t)p.batch * p.max_pages_per_req;
  for (int64_t e = tid; e < pairs; e += kValidateThreads) {
    const int b = (int)(e / p.max_pages_per_req), pg = (int)(e - (int64_t)b * p.max_pages_per_req);
    const int len = p.ctx_lens[b];
    if (len > 0 && pg < (len + kPage - 1) / kPage) {
      const int id = p.block_table[e];
      if (id < 0 || id >= p.num_pages) f |= kValidPageId;
    }
  }
  if (f) atomicOr(&flags, f);
  __syncthreads();
  if (tid == 0) *p.error_word = flags;
}

}  // namespace dsa

using namespace dsa;

hipError_t dsa_launch_validate(const int32_t* q_offsets, const int32_t* ctx_lens, const int32_t* block_table,
                               int batch, int num_q_tokens, int max_q_per_req, int max_ctx_len,
                               int max_pages_per_req, int num_pages, uint32_t* error_word, hipStream_t s) {
  ValidateParams p{q_offsets, ctx_lens, block_table, batch, num_q_tokens, max_q_per_req, max_ctx_len,
                   max_pages_per_req, num_pages, error_word};
  hipLaunchKernelGGL(validate_paged, dim3(1), dim3(kValidateThreads), 0, s, p);
  return hipGetLastError();
}
