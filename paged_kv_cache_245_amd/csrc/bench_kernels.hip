// bench_kernels.hip - measurement kernels: a plain 16-byte-per-lane copy (known
// traffic, used to calibrate hardware byte counters), a streaming read (the
// achievable HBM read ceiling), a buffer overwrite that evicts the last-level
// cache between timed runs, and a dense bf16 MFMA loop on caller-supplied
// operands (the matrix-core rate the chip sustains on such data).
#include <algorithm>

#include "pa_device.h"

namespace pa {
namespace {

constexpr int kThreads = 256;

unsigned grid_for(size_t n16) {
  size_t b = (n16 + kThreads - 1) / kThreads;
  if (b > 8192) b = 8192;
  if (b == 0) b = 1;
  return (unsigned)b;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(u32x4* __restrict__ dst,
                                                        const u32x4* __restrict__ src,
                                                        int64_t n16) {
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += step)
    dst[i] = src[i];
}

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src,
                                                        int64_t n16, float* __restrict__ sink) {
  // eight independent non-temporal 16-byte loads in flight per lane per iteration;
  // launched with one workgroup (four wavefronts) per compute unit. A sweep of
  // 1-16 loads in flight, 4-32 wavefronts per compute unit and plain or
  // non-temporal loads over 4 GiB put this shape at the top (about 7.1 TB/s).
  const int64_t step = (int64_t)gridDim.x * kThreads;
  uint32_t x = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 7 * step < n16; i += 8 * step) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * step);
#pragma unroll
    for (int u = 0; u < 8; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += step) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = x;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] ^= red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x % 4096] = __uint_as_float(red[0] & 0x007fffffu);
}

__global__ __launch_bounds__(kThreads) void flush_kernel(u32x4* __restrict__ buf, int64_t n16) {
  const int64_t step = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += step) {
    const uint32_t x = (uint32_t)i;
    buf[i] = u32x4{x, x ^ 0x55555555u, x + 1u, ~x};
  }
}

// MFMA 32x32x16 bf16 on every SIMD: 8 wavefronts per workgroup, each lane holding
// 8 operand fragments of 16 bytes read once from `operands` (fragment i of thread
// t of workgroup b at [(b * 512 + t) * 8 + i]), then `iters` rounds of 8 products
// into 4 independent accumulators; each thread writes one checksum float.
__global__ __launch_bounds__(512) void mfma_kernel(const u32x4* __restrict__ operands, int iters,
                                                   float* __restrict__ sink) {
  const int64_t t = (int64_t)blockIdx.x * 512 + threadIdx.x;
  bf16x8 fa[4], fb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[i] = as_bf16x8(operands[t * 8 + i]);
    fb[i] = as_bf16x8(operands[t * 8 + 4 + i]);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[(2 * j) & 3], fb[(2 * j + 1) & 3], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[(2 * j + 1) & 3], fb[(2 * j + 2) & 3], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[(2 * j + 2) & 3], fb[(2 * j + 3) & 3], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[(2 * j + 3) & 3], fb[(2 * j) & 3], c3, 0, 0, 0);
    }
  }
  float x = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) x += c0[i] + c1[i] + c2[i] + c3[i];
  sink[t] = x;
}

}  // namespace

hipError_t launch_bench_mfma(const void* operands, int workgroups, int iters, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_kernel, dim3(workgroups), dim3(512), 0, stream, (const u32x4*)operands, iters, sink);
  return hipGetLastError();
}

hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, (u32x4*)dst,
                     (const u32x4*)src, n);
  return hipGetLastError();
}

hipError_t launch_bench_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  const unsigned grid = std::min<unsigned>(grid_for(n), (unsigned)std::max(cus, 1));
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kThreads), 0, stream, (const u32x4*)src, n, sink);
  return hipGetLastError();
}

hipError_t launch_bench_flush(void* buf, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(flush_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, (u32x4*)buf, n);
  return hipGetLastError();
}

}  // namespace pa
