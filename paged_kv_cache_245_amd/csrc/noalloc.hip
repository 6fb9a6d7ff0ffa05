// noalloc.hip - pa_decode_append_noalloc: pa_decode_append with its split-KV
// workspace taken from a fixed device array of this library instead of a buffer
// the caller allocates, for callers that cannot allocate device memory (work
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). The kernels are pa_decode_append's; only the workspace differs.
//
// `scratch` below exists once per GPU the library runs on, for the life of the
// process. In host code its name is a host-side stand-in, not a device address:
// the device address of each GPU's copy is looked up once per device, with that
// device current, and only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "pa.h"
#include "pa_device.h"

static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up
std::mutex g_scratch_mu;                    // serialises the first lookups

// Device address of the current device's `scratch`; PA_OK or a negative status.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return pa::set_error_detail(PA_ERR_HIP, (std::string("hipGetDevice: ") + hipGetErrorString(e)).c_str());
  }
  if (dev < 0 || dev >= kMaxDevices)
    return pa::set_error_detail(PA_ERR_UNSUPPORTED, "device index above 63");
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return pa::set_error_detail(
            PA_ERR_HIP, (std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e)).c_str());
      }
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode_append_noalloc(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                             const void* value, void* k_cache, void* v_cache, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len, float scale, int32_t partition_tokens, void* stream) {
  if (num_seqs <= 0 || desc == nullptr)  // no-op, or an argument error pa_decode_append names
    return pa_decode_append(desc, out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq,
                            context_lens, num_seqs, max_context_len, scale, partition_tokens, nullptr, 0,
                            stream);
  if (!out || !q || !key || !value || !k_cache || !v_cache || !block_tables || !context_lens)
    return pa::set_error_detail(PA_ERR_INVALID_ARG, "null pointer argument");
  const size_t need = pa_decode_workspace_size(desc, num_seqs, max_context_len, partition_tokens);
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return pa::set_error_detail(
        PA_ERR_WORKSPACE,
        ("pa_decode_append_noalloc: these sizes need " + std::to_string(need) +
         " bytes of workspace, more than the library's fixed " + std::to_string(PA_NOALLOC_SCRATCH_BYTES) +
         " bytes; use pa_decode_append with a workspace of that size")
            .c_str());
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st != PA_OK) return st;
  }
  return pa_decode_append(desc, out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq,
                          context_lens, num_seqs, max_context_len, scale, partition_tokens, ws,
                          ws ? (size_t)PA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

}  // extern "C"
