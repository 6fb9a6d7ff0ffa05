// write_kv.hip - store new tokens' K/V rows into their pool slots.
//
// The KV cache grows one token at a time; each new token's K and V rows are
// written once into the slot its request's block table assigns (block * 16 +
// offset), then read by every later token (arcyou teardown of vLLM paged
// attention, sections "The problem both ideas solve" and "PagedAttention: the
// KV cache is paged, like virtual memory").
//
// One thread moves one 16-byte piece of a token's row for K and for V. A
// token's row (all kv heads) is contiguous both in the input and in the pool,
// so a wavefront reads and writes whole rows: 2 KiB per token for 8 kv heads x
// 128 bf16. The copy is bit-exact and HBM-bound.
#include "pa_device.h"

namespace pa {
namespace {

__global__ __launch_bounds__(256) void write_kv_kernel(const u32x4* __restrict__ key,
                                                       const u32x4* __restrict__ value,
                                                       u32x4* __restrict__ k_cache,
                                                       u32x4* __restrict__ v_cache,
                                                       const int32_t* __restrict__ slots,
                                                       int64_t num_tokens, int pieces_per_row,
                                                       int64_t num_slots) {
  const int64_t total = num_tokens * pieces_per_row;
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += step) {
    const int64_t tok = i / pieces_per_row;
    const int piece = (int)(i - tok * pieces_per_row);
    const int32_t slot = slots[tok];
    if (slot < 0 || (int64_t)slot >= num_slots) continue;  // -1 = skip; out of range = skip
    // kv_row with one "head" whose width is the whole row in 16-byte pieces
    const int64_t dst = kv_row(slot >> 4, slot & 15, 0, 1, pieces_per_row) + piece;
    const u32x4 kk = __builtin_nontemporal_load(key + i);
    const u32x4 vv = __builtin_nontemporal_load(value + i);
    k_cache[dst] = kk;
    v_cache[dst] = vv;
  }
}

// Each request's newest token at position context_len - 1, stored through the
// request's block table (one workgroup per request, 16-byte pieces of the row).
__global__ __launch_bounds__(256) void append_kv_kernel(const u32x4* __restrict__ key,
                                                        const u32x4* __restrict__ value,
                                                        u32x4* __restrict__ k_cache,
                                                        u32x4* __restrict__ v_cache,
                                                        const int32_t* __restrict__ block_tables,
                                                        int32_t max_blocks,
                                                        const int32_t* __restrict__ context_lens,
                                                        int32_t max_context_len, int pieces_per_row,
                                                        int64_t num_blocks) {
  const int s = blockIdx.x;
  const int L = min(context_lens[s], max_context_len);
  if (L < 1) return;
  const int32_t id = block_tables[(int64_t)s * max_blocks + ((L - 1) >> 4)];
  if (!block_ok(id, num_blocks)) return;
  const int64_t dst = kv_row(id, (L - 1) & 15, 0, 1, pieces_per_row);
  for (int i = threadIdx.x; i < pieces_per_row; i += blockDim.x) {
    k_cache[dst + i] = key[(int64_t)s * pieces_per_row + i];
    v_cache[dst + i] = value[(int64_t)s * pieces_per_row + i];
  }
}

}  // namespace

hipError_t launch_append_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int row_bytes, int64_t num_blocks,
                            hipStream_t stream) {
  hipLaunchKernelGGL(append_kv_kernel, dim3((unsigned)num_seqs), dim3(256), 0, stream, (const u32x4*)key,
                     (const u32x4*)value, (u32x4*)k_cache, (u32x4*)v_cache, block_tables, max_blocks,
                     context_lens, max_context_len, row_bytes / 16, num_blocks);
  return hipGetLastError();
}

hipError_t launch_write_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int32_t* slots, int64_t num_tokens, int row_bytes,
                           int64_t num_slots, hipStream_t stream) {
  const int pieces = row_bytes / 16;
  const int64_t total = num_tokens * pieces;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(write_kv_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const u32x4*)key, (const u32x4*)value, (u32x4*)k_cache, (u32x4*)v_cache,
                     slots, num_tokens, pieces, num_slots);
  return hipGetLastError();
}

}  // namespace pa
