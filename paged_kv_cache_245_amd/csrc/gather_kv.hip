// gather_kv.hip - copy each request's logical K/V out of the pool through its
// block table (inspection aid). It addresses the pool with the same kv_row()
// and table_block() helpers as the attention kernels, so a bit-exact match
// with the oracle's gather checks the indexing those kernels rely on: logical
// token t of a request lives in block table[t / 16] at offset t % 16 (arcyou
// teardown of vLLM paged attention, section "PagedAttention: the KV cache is
// paged, like virtual memory").
#include "pa_device.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void gather_kv_kernel(u32x4* __restrict__ dst_k,
                                                        u32x4* __restrict__ dst_v,
                                                        const u32x4* __restrict__ k_cache,
                                                        const u32x4* __restrict__ v_cache,
                                                        const int32_t* __restrict__ tables,
                                                        int32_t max_blocks,
                                                        const int32_t* __restrict__ lens,
                                                        int32_t max_context_len,
                                                        int pieces_per_row, int64_t num_blocks) {
  const int s = blockIdx.y;
  int L = lens[s];
  L = min(L, max_context_len);
  if (L <= 0) return;
  const int32_t* row = tables + (int64_t)s * max_blocks;
  const int64_t total = (int64_t)L * pieces_per_row;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int t = (int)(i / pieces_per_row);
    const int piece = (int)(i - (int64_t)t * pieces_per_row);
    const int32_t id = table_block(row, t);
    if (!block_ok(id, num_blocks)) continue;
    const int64_t src = kv_row(id, t & 15, 0, 1, pieces_per_row) + piece;
    const int64_t dst = ((int64_t)s * max_context_len + t) * pieces_per_row + piece;
    dst_k[dst] = k_cache[src];
    dst_v[dst] = v_cache[src];
  }
}

}  // namespace

hipError_t launch_gather_kv(void* dst_k, void* dst_v, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int row_bytes, int num_kv_heads,
                            int64_t num_blocks, hipStream_t stream) {
  (void)num_kv_heads;
  const int pieces = row_bytes / 16;
  const int64_t per_seq = (int64_t)max_context_len * pieces;
  int64_t bx = (per_seq + 255) / 256;
  if (bx > 4096) bx = 4096;
  hipLaunchKernelGGL(gather_kv_kernel, dim3((unsigned)bx, (unsigned)num_seqs), dim3(256), 0,
                     stream, (u32x4*)dst_k, (u32x4*)dst_v, (const u32x4*)k_cache,
                     (const u32x4*)v_cache, block_tables, max_blocks, context_lens,
                     max_context_len, pieces, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
