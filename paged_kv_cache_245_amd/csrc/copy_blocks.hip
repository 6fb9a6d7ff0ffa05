// copy_blocks.hip - duplicate whole K/V blocks inside the pool (copy-on-write).
//
// Forked sequences share physical blocks until one of them must write into a
// shared block; that block is duplicated first and the writer's table points
// at the copy (aitrending, "The 1960s Operating System Trick That Makes vLLM 4x
// Faster", section Technical Details). One workgroup copies one (source,
// destination) pair for K and V with 16-byte lanes; a block is contiguous
// (16 tokens x all kv heads), so the copy is a straight stream. HBM-bound.
//
// swap_blocks_kernel moves blocks between the device pool and a swap pool in
// pinned host memory (swap-out on preemption, swap-in on resumption: same page,
// Technical Details). Same shape of work; bound by the host link.
#include "pa_device.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(u32x4* __restrict__ k_cache,
                                                               u32x4* __restrict__ v_cache,
                                                               const int32_t* __restrict__ pairs,
                                                               int row_pieces, int64_t num_blocks) {
  const int32_t src = pairs[2 * (int64_t)blockIdx.x];
  const int32_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if (!block_ok(src, num_blocks) || !block_ok(dst, num_blocks)) return;  // skipped
  // a token row is row_pieces 16-byte pieces (all kv heads); a block is 16 rows
  const int64_t s0 = kv_row(src, 0, 0, 1, row_pieces), d0 = kv_row(dst, 0, 0, 1, row_pieces);
  for (int i = threadIdx.x; i < kBlock * row_pieces; i += kThreads) {
    const u32x4 kk = __builtin_nontemporal_load(k_cache + s0 + i);
    const u32x4 vv = __builtin_nontemporal_load(v_cache + s0 + i);
    k_cache[d0 + i] = kk;
    v_cache[d0 + i] = vv;
  }
}

// One workgroup per pair; the host side is read or written through the
// device-visible address of pinned host memory.
__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(u32x4* __restrict__ k_cache,
                                                               u32x4* __restrict__ v_cache,
                                                               u32x4* __restrict__ host_k,
                                                               u32x4* __restrict__ host_v,
                                                               const int32_t* __restrict__ pairs,
                                                               int row_pieces, int64_t num_blocks,
                                                               int64_t num_host_blocks, bool to_host) {
  const int32_t a = pairs[2 * (int64_t)blockIdx.x];
  const int32_t b = pairs[2 * (int64_t)blockIdx.x + 1];
  const int32_t dev = to_host ? a : b, hst = to_host ? b : a;
  if (!block_ok(dev, num_blocks) || !block_ok(hst, num_host_blocks)) return;  // skipped
  const int64_t d0 = kv_row(dev, 0, 0, 1, row_pieces), h0 = kv_row(hst, 0, 0, 1, row_pieces);
  for (int i = threadIdx.x; i < kBlock * row_pieces; i += kThreads) {
    if (to_host) {
      const u32x4 kk = __builtin_nontemporal_load(k_cache + d0 + i);
      const u32x4 vv = __builtin_nontemporal_load(v_cache + d0 + i);
      host_k[h0 + i] = kk;
      host_v[h0 + i] = vv;
    } else {
      const u32x4 kk = host_k[h0 + i];
      const u32x4 vv = host_v[h0 + i];
      k_cache[d0 + i] = kk;
      v_cache[d0 + i] = vv;
    }
  }
}

}  // namespace

hipError_t launch_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v,
                              const int32_t* pairs, int64_t num_pairs, int64_t block_bytes,
                              int64_t num_blocks, int64_t num_host_blocks, bool to_host,
                              hipStream_t stream) {
  const int row_pieces = (int)(block_bytes / 16 / kBlock);
  hipLaunchKernelGGL(swap_blocks_kernel, dim3((unsigned)num_pairs), dim3(kThreads), 0, stream,
                     (u32x4*)k_cache, (u32x4*)v_cache, (u32x4*)host_k, (u32x4*)host_v, pairs,
                     row_pieces, num_blocks, num_host_blocks, to_host);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int64_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream) {
  const int row_pieces = (int)(block_bytes / 16 / kBlock);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)num_pairs), dim3(kThreads), 0, stream,
                     (u32x4*)k_cache, (u32x4*)v_cache, pairs, row_pieces, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
