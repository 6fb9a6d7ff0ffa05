// pa_device.h - device helpers shared by the gfx950 kernels, and the internal
// launcher interface between the kernels and the C ABI in pa_api.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kBlock = 16;  // tokens per physical KV block

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Element offset of the K/V row of (physical block, offset in block, kv head).
// Every kernel that reads or writes the pool addresses it through this function.
__device__ __forceinline__ int64_t kv_row(int32_t block_id, int offset, int kv_head,
                                          int num_kv_heads, int head_dim) {
  return ((int64_t)block_id * kBlock + offset) * (int64_t)(num_kv_heads * head_dim) +
         (int64_t)kv_head * head_dim;
}

// Physical block holding logical token t of a request (its block-table row);
// the caller range-checks the id before addressing the pool with it.
__device__ __forceinline__ int32_t table_block(const int32_t* table_row, int t) {
  return table_row[t >> 4];
}

__device__ __forceinline__ bool block_ok(int32_t id, int64_t num_blocks) {
  return id >= 0 && (int64_t)id < num_blocks;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float -> bfloat16 bits, round to nearest with ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two floats -> packed bf16 pair (low half = a), hardware round-to-nearest-even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- launchers
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* part_acc;  // [S][Hq][max_parts][D] (bf16 values, D per row, in shared-prefix mode)
  float* part_ml;   // [S][Hq][max_parts][2]: running max (log2 units), sum of exponentials
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t max_context_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t partition_tokens;  // fixed-partition mode: keys per partition
  int32_t max_parts;         // fixed-partition mode: partitions of the longest request
  int32_t num_workers;       // balanced mode: workgroups along the block axis (0 = fixed mode)
  int32_t nontemporal;       // stream K/V past the caches: 1 yes, 0 no, -1 kernel decides
  int32_t* cum_blocks;       // balanced mode: [S+1] prefix sums of blocks per request
  // balanced mode: [num_workers] the request whose first cut between two workers
  // falls at the start of this worker's range, or -1 (each split request once)
  int32_t* split_req;
  int32_t merge_splits;      // balanced merge grid runs over split_req instead of requests
  int32_t lean;              // balanced mode: the lean decode kernel (one wavefront per workgroup)
  int32_t ring_bytes;        // balanced mode: LDS bytes per wavefront for staged segment results
                             // (set at launch; 0 = each segment stores its result directly)
  // Short-chunk mode (balanced bf16, pa_prefill_chunk_short; null and 0 otherwise): request s
  // has query_start_loc[s+1] - query_start_loc[s] <= n_cols new tokens, its q rows from
  // query_start_loc[s], all of them already in the pool (context_lens holds seq_lens).
  // Column n of a kv head's score tile is (position n / group, q head n % group), and
  // position p attends the keys before context_len - new tokens + p + 1.
  const int32_t* query_start_loc;
  int32_t n_cols;
  float scale_log2;  // scale * log2(e)
  // Append mode (balanced bf16 only; both null otherwise): [S][Hkv][D] K and V of
  // each request's newest token, position context_len - 1. The decode kernel
  // reads only the keys before it from the pool; the merge attends it from here
  // and stores it into its slot through the block table.
  const void* new_k;
  const void* new_v;
  // Shared-prefix mode (balanced only): every request's first skip_blocks blocks
  // are not read; every segment leaves a partial (partial_only); and the merge
  // also folds pre_parts partials per (request, q head) from pre_acc / pre_ml
  // (laid out as PrefillArgs' part_acc / part_ml; the accumulators in bf16).
  int32_t skip_blocks;
  int32_t partial_only;
  int32_t pre_parts;
  const uint16_t* pre_acc;
  const float* pre_ml;
};

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  const int32_t* query_start_loc;
  const int32_t* seq_lens;
  const int32_t* block_tables;
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_query_len;
  int32_t max_seq_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  float scale_log2;
  // Shared-prefix mode (launch_prefix_attention): the rows are the decode
  // queries q [num_seqs][Hq][D], all attending the first prefix_keys keys of
  // block table row 0 with no causal mask; the keys are split into key_splits
  // ranges of key_chunk (a multiple of 64), and each (request, q head, range)
  // leaves a partial (m, l, acc) instead of an output. acc (the weighted sum of
  // V rows, not divided by l) is stored in bf16, rounded to nearest even, as the
  // outputs are: it halves the bytes the pass writes and the merge reads.
  int32_t prefix_keys;
  int32_t key_chunk;
  int32_t key_splits;
  uint16_t* part_acc;  // [num_seqs][Hq][key_splits][D] bf16
  float* part_ml;      // [num_seqs][Hq][key_splits][2]
  // Append mode (launch_prefill with both set): [num_tokens][Hkv][D] K and V of
  // the chunks' own tokens, row t for query row t. The kernel reads a chunk's keys
  // from here instead of the pool, and each workgroup stores the rows of its own
  // query positions into the pool (k, v) through the block table.
  const uint16_t* new_k;
  const uint16_t* new_v;
};

// Records `what` as the detail of the calling thread's last error (returned by
// pa_last_error_detail) and returns `status`.
int set_error_detail(int status, const char* what);

hipError_t launch_write_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                           const int32_t* slots, int64_t num_tokens, int row_bytes,
                           int64_t num_slots, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int head_dim, bool bf16, hipStream_t stream);
// Stores each request's newest K/V row ([S][Hkv][D], position context_len - 1)
// into its slot through the block table; requests with length < 1 or a bad
// block id are skipped.
hipError_t launch_append_kv(const void* key, const void* value, void* k_cache, void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks, const int32_t* context_lens,
                            int32_t num_seqs, int32_t max_context_len, int row_bytes, int64_t num_blocks,
                            hipStream_t stream);
// kv heads handled by one decode workgroup (one wavefront each)
int decode_waves(int num_kv_heads);
// most requests the balanced decode mode accepts (block prefix sums live in LDS)
int decode_max_balanced_seqs();
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int group, hipStream_t stream);
hipError_t launch_prefix_attention(const PrefillArgs& a, int head_dim, int group, hipStream_t stream);
hipError_t launch_gather_kv(void* dst_k, void* dst_v, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t max_context_len, int row_bytes, int num_kv_heads,
                            int64_t num_blocks, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int64_t num_pairs,
                              int64_t block_bytes, int64_t num_blocks, hipStream_t stream);
// Copies whole blocks between the device pool and a host swap pool (pointers the
// device can address); to_host: pairs are (device, host), else (host, device).
hipError_t launch_swap_blocks(void* k_cache, void* v_cache, void* host_k, void* host_v,
                              const int32_t* pairs, int64_t num_pairs, int64_t block_bytes,
                              int64_t num_blocks, int64_t num_host_blocks, bool to_host,
                              hipStream_t stream);
hipError_t launch_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_bench_read(const void* src, size_t bytes, float* sink, hipStream_t stream);
hipError_t launch_bench_flush(void* buf, size_t bytes, hipStream_t stream);
hipError_t launch_bench_mfma(const void* operands, int workgroups, int iters, float* sink, hipStream_t stream);

}  // namespace pa
