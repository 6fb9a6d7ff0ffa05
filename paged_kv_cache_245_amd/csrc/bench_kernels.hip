// bench_kernels.hip - measurement kernels: a plain 16-byte-per-lane copy (known
// traffic, used to calibrate hardware byte counters), a streaming read (the
// achievable HBM read ceiling), and a buffer overwrite that evicts the
// last-level cache between timed runs.
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
  // four independent 16-byte loads in flight per lane per iteration
  const int64_t step = (int64_t)gridDim.x * kThreads;
  uint32_t x = 0;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * step < n16; i += 4 * step) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + step);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * step);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * step);
    x ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^
         d[0] ^ d[1] ^ d[2] ^ d[3];
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

}  // namespace

hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, (u32x4*)dst,
                     (const u32x4*)src, n);
  return hipGetLastError();
}

hipError_t launch_bench_read(const void* src, size_t bytes, float* sink, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(read_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream,
                     (const u32x4*)src, n, sink);
  return hipGetLastError();
}

hipError_t launch_bench_flush(void* buf, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 16);
  hipLaunchKernelGGL(flush_kernel, dim3(grid_for(n)), dim3(kThreads), 0, stream, (u32x4*)buf, n);
  return hipGetLastError();
}

}  // namespace pa
