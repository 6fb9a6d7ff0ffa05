// pa_api.hip - the C ABI declared in include/pa.h: argument validation, the
// optional host-side content check (PA_CHECK=1), split-KV sizing, and kernel
// dispatch on the caller's stream. No device memory is allocated here.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <string>
#include <unordered_set>
#include <vector>

#include "pa.h"
#include "pa_device.h"

namespace {

thread_local std::string g_detail;

int fail(int status, const std::string& what) {
  g_detail = what;
  return status;
}

bool check_mode() {  // read on every call, so a process can switch it on and off
  const char* e = std::getenv("PA_CHECK");
  return e != nullptr && e[0] == '1';
}

int elem_bytes(int32_t dtype) { return dtype == PA_BF16 ? 2 : 4; }

int validate_desc(const pa_cache_desc* d) {
  if (d == nullptr) return fail(PA_ERR_INVALID_ARG, "desc is NULL");
  if (d->reserved != 0) return fail(PA_ERR_INVALID_ARG, "desc.reserved must be 0");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0)
    return fail(PA_ERR_INVALID_ARG, "head counts must be positive");
  if (d->num_q_heads % d->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  if (d->num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "num_blocks must be positive");
  if (d->num_blocks > (int64_t)INT32_MAX / PA_BLOCK_SIZE)
    return fail(PA_ERR_UNSUPPORTED, "num_blocks * 16 must fit in int32 slots");
  if (d->block_size != PA_BLOCK_SIZE) return fail(PA_ERR_UNSUPPORTED, "block_size must be 16");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->dtype != PA_F32 && d->dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "unknown dtype");
  const int g = d->num_q_heads / d->num_kv_heads;
  if (d->dtype == PA_BF16 && g != 1 && g != 2 && g != 4 && g != 8 && g != 16)
    return fail(PA_ERR_UNSUPPORTED, "bf16 kernels need q heads per kv head in {1,2,4,8,16}");
  if (d->dtype == PA_F32 && g > 16)
    return fail(PA_ERR_UNSUPPORTED, "fp32 kernels need at most 16 q heads per kv head");
  return PA_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PA_OK;
  return fail(PA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

template <class T>
bool fetch(std::vector<T>& host, const void* dev, size_t count) {
  host.resize(count);
  if (count == 0) return true;
  return hipMemcpy(host.data(), dev, count * sizeof(T), hipMemcpyDeviceToHost) == hipSuccess;
}

// Check that the blocks holding tokens 0..len-1 of every request are in the pool.
int check_tables(const std::vector<int32_t>& tables, int32_t max_blocks,
                 const std::vector<int32_t>& lens, int64_t num_blocks) {
  for (size_t s = 0; s < lens.size(); ++s) {
    const int nb = (lens[s] + PA_BLOCK_SIZE - 1) / PA_BLOCK_SIZE;
    for (int b = 0; b < nb; ++b) {
      const int32_t id = tables[s * (size_t)max_blocks + b];
      if (id < 0 || id >= num_blocks)
        return fail(PA_ERR_RANGE, "block_tables[" + std::to_string(s) + "][" + std::to_string(b) +
                                      "] = " + std::to_string(id) + " is outside the pool");
    }
  }
  return PA_OK;
}

int32_t env_partition() {
  const char* e = std::getenv("PA_PARTITION_TOKENS");
  if (e == nullptr) return 0;
  const int v = std::atoi(e);
  return (v > 0 && v % PA_BLOCK_SIZE == 0) ? v : 0;
}

// Partition size: the largest of 4096..256 keys that still yields at least
// ~16 wavefronts per compute unit (256 CUs) if every request had the maximum
// length; at least 256 keys, and no split when one partition covers all.
int32_t choose_partition(const pa_cache_desc* d, int32_t num_seqs, int32_t max_context_len) {
  const int32_t forced = env_partition();
  if (forced > 0) return forced;
  const int64_t target = 4096;
  const int64_t units = (int64_t)num_seqs * d->num_kv_heads;
  for (int32_t p = 4096; p >= 256; p >>= 1) {
    const int64_t parts = ((int64_t)max_context_len + p - 1) / p;
    if (units * parts >= target) return p;
  }
  return 256;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int env_int(const char* name, int dflt) {
  const char* e = std::getenv(name);
  return e != nullptr ? std::atoi(e) : dflt;
}

// Compute units of the calling thread's current device, read once per device
// (256 on MI355X). The decode's worker counts derive from it; a device the
// runtime cannot name is taken to have 256.
constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];

int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int n = g_cus[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

// Balanced decode: enough workgroups for eight wavefronts per compute unit
// (2,048 on a 256-CU MI355X), each wavefront one kv head of one workgroup.
int32_t balanced_workers(const pa_cache_desc* d) {
  const int forced = env_int("PA_DECODE_WORKERS", 0);  // tuning override
  if (forced > 0) return forced;
  const int nw = pa::decode_waves(d->num_kv_heads);
  const int groups = (d->num_kv_heads + nw - 1) / nw;
  const int w = 8 * device_cus() / (nw * groups);
  return w > 0 ? w : 1;
}

// Lean decode: one wavefront per SIMD (four per compute unit; 1,024 on a 256-CU
// MI355X), each a kv head of one workgroup.
int32_t lean_workers(const pa_cache_desc* d) {
  const int forced = env_int("PA_DECODE_LEAN_WORKERS", 0);  // tuning override
  if (forced > 0) return forced;
  return std::max(1, 4 * device_cus() / d->num_kv_heads);
}

struct DecodeLayout {
  int32_t partition;  // fixed mode
  int32_t max_parts;  // fixed mode
  int32_t workers;    // balanced mode (0 = fixed mode)
  size_t acc_bytes;
  size_t ml_bytes;
  size_t total;
};

DecodeLayout decode_layout(const pa_cache_desc* d, int32_t num_seqs, int32_t max_context_len,
                           int32_t partition_tokens) {
  DecodeLayout l{};
  size_t rows = 0;
  if (d->dtype == PA_BF16 && partition_tokens == 0 && num_seqs <= pa::decode_max_balanced_seqs()) {
    l.workers = balanced_workers(d);
    rows = ((size_t)num_seqs + l.workers) * d->num_q_heads;
  } else {
    l.partition = partition_tokens > 0 ? partition_tokens
                                       : choose_partition(d, num_seqs, max_context_len);
    l.max_parts = (int32_t)(((int64_t)max_context_len + l.partition - 1) / l.partition);
    if (l.max_parts <= 1) return l;
    rows = (size_t)num_seqs * d->num_q_heads * l.max_parts;
  }
  l.acc_bytes = align256(rows * d->head_dim * sizeof(float));
  l.ml_bytes = align256(rows * 2 * sizeof(float));
  l.total = l.acc_bytes + l.ml_bytes;
  // balanced mode: the block prefix sums [S+1], then the split-request records [workers]
  if (l.workers > 0) l.total += align256(((size_t)num_seqs + 1 + l.workers) * sizeof(int32_t));
  return l;
}

// Short chunks through the balanced decode: its workspace with one partial row
// per (request + worker, position, q head), positions up to max_query_len.
DecodeLayout chunk_short_layout(const pa_cache_desc* d, int32_t num_seqs, int32_t max_query_len) {
  DecodeLayout l{};
  l.workers = balanced_workers(d);
  const size_t rows = ((size_t)num_seqs + l.workers) * (size_t)max_query_len * d->num_q_heads;
  l.acc_bytes = align256(rows * d->head_dim * sizeof(float));
  l.ml_bytes = align256(rows * 2 * sizeof(float));
  l.total = l.acc_bytes + l.ml_bytes + align256(((size_t)num_seqs + 1 + l.workers) * sizeof(int32_t));
  return l;
}

// Shared-prefix decode: the balanced decode's workspace (for the tails), then the
// prefix pass's partials [S][Hq][splits][D] and [S][Hq][splits][2]. The prefix
// keys are split into ranges of whole 64-key tiles so that the prefix pass has
// about one workgroup (256 packed rows of one kv head) per two compute units:
// that timed as one per compute unit did and leaves half the partials, which
// the merge reads back; more, shorter ranges paid their set-up twice.
struct PrefixLayout {
  DecodeLayout dec;
  int32_t key_chunk;
  int32_t splits;
  size_t acc_offset, ml_offset, total;
};

PrefixLayout prefix_layout(const pa_cache_desc* d, int32_t num_seqs, int32_t max_context_len,
                           int32_t prefix_blocks) {
  PrefixLayout p{};
  p.dec = decode_layout(d, num_seqs, max_context_len, 0);
  const int64_t keys = (int64_t)prefix_blocks * PA_BLOCK_SIZE;
  const int64_t tiles = (keys + 63) / 64;
  const int group = d->num_q_heads / d->num_kv_heads;
  const int64_t row_tiles = ((int64_t)num_seqs * group + 255) / 256;
  const int64_t wgs = (int64_t)d->num_kv_heads * row_tiles;
  const int64_t target = std::max(1, env_int("PA_PREFIX_WORKGROUPS", device_cus() / 2));  // tuning override
  int64_t splits = std::min<int64_t>(std::max<int64_t>(tiles, 1), std::max<int64_t>(1, (target + wgs - 1) / wgs));
  const int64_t tiles_per = (tiles + splits - 1) / splits;
  p.key_chunk = (int32_t)(64 * std::max<int64_t>(tiles_per, 1));
  p.splits = (int32_t)std::max<int64_t>(1, (keys + p.key_chunk - 1) / p.key_chunk);
  const size_t rows = (size_t)num_seqs * d->num_q_heads * p.splits;
  p.acc_offset = align256(p.dec.total);
  p.ml_offset = p.acc_offset + align256(rows * d->head_dim * sizeof(uint16_t));  // bf16 accumulators
  p.total = p.ml_offset + align256(rows * 2 * sizeof(float));
  return p;
}

// Non-temporal K/V loads: -1 lets the balanced kernel decide from the total
// attended blocks; the fixed-partition kernel streams when no block can be read
// twice and the pool is far larger than the 256 MiB last-level cache.
int32_t nontemporal_mode(const pa_cache_desc* d, int32_t num_seqs, int32_t max_context_len,
                         bool balanced) {
  const int forced = env_int("PA_DECODE_NT", -1);
  if (forced >= 0) return forced != 0;
  if (balanced) return -1;
  const int64_t pool_tokens = d->num_blocks * PA_BLOCK_SIZE;
  const int64_t pool_bytes = 2 * pool_tokens * d->num_kv_heads * d->head_dim * elem_bytes(d->dtype);
  return (int64_t)num_seqs * max_context_len <= pool_tokens && pool_bytes >= ((int64_t)1 << 30);
}

}  // namespace

namespace pa {
int set_error_detail(int status, const char* what) { return fail(status, what); }
}  // namespace pa

extern "C" {

int pa_version(void) { return PA_VERSION; }

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_ERR_WORKSPACE: return "decode workspace missing or too small";
    case PA_ERR_RANGE: return "metadata out of range (check mode)";
    case PA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* pa_last_error_detail(void) { return g_detail.c_str(); }

int pa_write_kv(const pa_cache_desc* desc, const void* key, const void* value, void* k_cache,
                void* v_cache, const int32_t* slot_mapping, int64_t num_tokens, void* stream) {
  int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (num_tokens < 0) return fail(PA_ERR_INVALID_ARG, "num_tokens is negative");
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  const int row_bytes = desc->num_kv_heads * desc->head_dim * elem_bytes(desc->dtype);
  const int64_t num_slots = desc->num_blocks * PA_BLOCK_SIZE;
  if (check_mode()) {
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess)
      return fail(PA_ERR_HIP, "stream synchronize failed");
    std::vector<int32_t> slots;
    if (!fetch(slots, slot_mapping, (size_t)num_tokens)) return fail(PA_ERR_HIP, "copy of slots failed");
    std::unordered_set<int32_t> seen;
    for (int64_t i = 0; i < num_tokens; ++i) {
      const int32_t s = slots[i];
      if (s == -1) continue;
      if (s < 0 || s >= num_slots)
        return fail(PA_ERR_RANGE, "slot_mapping[" + std::to_string(i) + "] = " + std::to_string(s) +
                                      " is outside the pool");
      if (!seen.insert(s).second)
        return fail(PA_ERR_RANGE, "slot " + std::to_string(s) + " is written twice");
    }
  }
  return hip_status(pa::launch_write_kv(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                        row_bytes, num_slots, as_stream(stream)),
                    "write_kv launch");
}

int32_t pa_decode_partition_tokens(const pa_cache_desc* desc, int32_t num_seqs,
                                   int32_t max_context_len) {
  int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (num_seqs < 0 || max_context_len < 0) return fail(PA_ERR_INVALID_ARG, "negative size");
  return choose_partition(desc, num_seqs, max_context_len);
}

size_t pa_decode_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                int32_t max_context_len, int32_t partition_tokens) {
  if (validate_desc(desc) != PA_OK || num_seqs <= 0 || max_context_len <= 0 ||
      partition_tokens < 0 || partition_tokens % PA_BLOCK_SIZE != 0)
    return 0;
  return decode_layout(desc, num_seqs, max_context_len, partition_tokens).total;
}

namespace {
// pa_decode; pa_decode_append when new_k/new_v are given; pa_decode_shared_prefix
// when prefix_blocks > 0 (balanced bf16 mode only).
int decode_impl(const pa_cache_desc* desc, void* out, const void* q, const void* new_k,
                const void* new_v, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                int32_t num_seqs, int32_t max_context_len, float scale, int32_t partition_tokens,
                void* workspace, size_t workspace_bytes, void* stream, int32_t prefix_blocks = 0,
                bool lean = false) {
  int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs is negative");
  if (num_seqs == 0) return PA_OK;
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs above 65535");
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  const bool append = new_k != nullptr || new_v != nullptr;
  if (append && (new_k == nullptr || new_v == nullptr))
    return fail(PA_ERR_INVALID_ARG, "key and value of the newest tokens are both needed");
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if (max_context_len <= 0) return fail(PA_ERR_INVALID_ARG, "max_context_len must be positive");
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE)
    return fail(PA_ERR_INVALID_ARG, "max_context_len exceeds 16 * max_blocks_per_seq");
  if (partition_tokens < 0 || partition_tokens % PA_BLOCK_SIZE != 0)
    return fail(PA_ERR_INVALID_ARG, "partition_tokens must be 0 or a positive multiple of 16");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  const bool prefix = prefix_blocks > 0;
  if (prefix) {
    if (desc->dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "a shared prefix needs a bf16 pool");
    if (num_seqs > pa::decode_max_balanced_seqs())
      return fail(PA_ERR_UNSUPPORTED, "a shared prefix needs at most 8192 requests");
    if ((int64_t)prefix_blocks * PA_BLOCK_SIZE > max_context_len)
      return fail(PA_ERR_INVALID_ARG, "prefix_blocks exceeds max_context_len / 16");
  }
  const PrefixLayout play = prefix_layout(desc, num_seqs, max_context_len, prefix ? prefix_blocks : 0);
  const DecodeLayout lay = prefix ? play.dec : decode_layout(desc, num_seqs, max_context_len, partition_tokens);
  const size_t need = prefix ? play.total : lay.total;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes");
  if (check_mode()) {
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess)
      return fail(PA_ERR_HIP, "stream synchronize failed");
    std::vector<int32_t> lens, tables;
    if (!fetch(lens, context_lens, num_seqs) ||
        !fetch(tables, block_tables, (size_t)num_seqs * max_blocks_per_seq))
      return fail(PA_ERR_HIP, "copy of metadata failed");
    for (int s = 0; s < num_seqs; ++s)
      if (lens[s] < 1 || lens[s] > max_context_len)
        return fail(PA_ERR_RANGE, "context_lens[" + std::to_string(s) + "] = " +
                                      std::to_string(lens[s]) + " is outside [1, max_context_len]");
    st = check_tables(tables, max_blocks_per_seq, lens, desc->num_blocks);
    if (st != PA_OK) return st;
    for (int s = 0; prefix && s < num_seqs; ++s) {
      if (lens[s] < prefix_blocks * PA_BLOCK_SIZE)
        return fail(PA_ERR_RANGE, "context_lens[" + std::to_string(s) + "] is shorter than the shared prefix");
      for (int b = 0; b < prefix_blocks; ++b)
        if (tables[(size_t)s * max_blocks_per_seq + b] != tables[b])
          return fail(PA_ERR_RANGE, "block_tables[" + std::to_string(s) + "][" + std::to_string(b) +
                                        "] differs from the shared prefix of row 0");
    }
  }
  pa::DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.part_acc = lay.total ? (float*)workspace : nullptr;
  a.part_ml = lay.total ? (float*)((char*)workspace + lay.acc_bytes) : nullptr;
  a.cum_blocks = lay.workers ? (int32_t*)((char*)workspace + lay.acc_bytes + lay.ml_bytes) : nullptr;
  a.split_req = lay.workers ? a.cum_blocks + num_seqs + 1 : nullptr;
  a.num_blocks = desc->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.max_context_len = max_context_len;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.group = desc->num_q_heads / desc->num_kv_heads;
  a.partition_tokens = lay.partition;
  a.max_parts = lay.max_parts;
  a.num_workers = lay.workers;
  if (lean && lay.workers > 0 && !prefix) {
    // one wavefront per workgroup and about four per compute unit (one per SIMD);
    // never more workers than the workspace was sized for
    a.lean = 1;
    a.num_workers = std::max(1, std::min<int32_t>(lay.workers, lean_workers(desc)));
  }
  a.nontemporal = nontemporal_mode(desc, num_seqs, max_context_len, lay.workers > 0);
  a.scale_log2 = scale * pa::kLog2e;
  if (prefix) {
    // the prefix once for all requests (MFMA, keys split into ranges), then the
    // tails through the balanced decode, both as partials for the merge
    pa::PrefillArgs pf{};
    pf.q = (const uint16_t*)q;
    pf.k = (const uint16_t*)k_cache;
    pf.v = (const uint16_t*)v_cache;
    pf.block_tables = block_tables;
    pf.num_blocks = desc->num_blocks;
    pf.max_blocks = max_blocks_per_seq;
    pf.num_seqs = num_seqs;
    pf.num_q_heads = desc->num_q_heads;
    pf.num_kv_heads = desc->num_kv_heads;
    pf.scale_log2 = a.scale_log2;
    pf.prefix_keys = prefix_blocks * PA_BLOCK_SIZE;
    pf.key_chunk = play.key_chunk;
    pf.key_splits = play.splits;
    pf.part_acc = (uint16_t*)((char*)workspace + play.acc_offset);
    pf.part_ml = (float*)((char*)workspace + play.ml_offset);
    st = hip_status(pa::launch_prefix_attention(pf, desc->head_dim, a.group, as_stream(stream)),
                    "prefix launch");
    if (st != PA_OK) return st;
    a.skip_blocks = prefix_blocks;
    a.partial_only = 1;
    a.pre_parts = play.splits;
    a.pre_acc = pf.part_acc;
    a.pre_ml = pf.part_ml;
  }
  if (append) {
    // Fused only when the requests do not outnumber the workers: then most
    // requests are split anyway and go through the merge, which takes the newest
    // token in. With more requests than workers most are whole, and writing
    // their output directly (after a small store of the newest tokens) is cheaper
    // than sending every request through the merge.
    if (lay.workers > 0 && desc->dtype == PA_BF16 && num_seqs <= a.num_workers) {
      a.new_k = new_k;  // the merge attends and stores the newest token
      a.new_v = new_v;
    } else {
      const int row_bytes = desc->num_kv_heads * desc->head_dim * elem_bytes(desc->dtype);
      st = hip_status(pa::launch_append_kv(new_k, new_v, const_cast<void*>(k_cache), const_cast<void*>(v_cache),
                                           block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                           max_context_len, row_bytes, desc->num_blocks, as_stream(stream)),
                      "append launch");
      if (st != PA_OK) return st;
    }
  }
  return hip_status(pa::launch_decode(a, desc->head_dim, desc->dtype == PA_BF16, as_stream(stream)),
                    "decode launch");
}
}  // namespace

int pa_decode(const pa_cache_desc* desc, void* out, const void* q, const void* k_cache,
              const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
              float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
              void* stream) {
  return decode_impl(desc, out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, scale, partition_tokens, workspace,
                     workspace_bytes, stream);
}

size_t pa_decode_shared_prefix_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                              int32_t max_context_len, int32_t prefix_blocks) {
  if (validate_desc(desc) != PA_OK || num_seqs <= 0 || max_context_len <= 0 || prefix_blocks < 0) return 0;
  if (prefix_blocks == 0) return decode_layout(desc, num_seqs, max_context_len, 0).total;
  return prefix_layout(desc, num_seqs, max_context_len, prefix_blocks).total;
}

int pa_decode_shared_prefix(const pa_cache_desc* desc, void* out, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                            int32_t prefix_blocks, float scale, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (prefix_blocks < 0) return fail(PA_ERR_INVALID_ARG, "prefix_blocks is negative");
  return decode_impl(desc, out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, scale, 0, workspace, workspace_bytes, stream,
                     prefix_blocks);
}

int pa_decode_append(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                     const void* value, void* k_cache, void* v_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                     int32_t max_context_len, float scale, int32_t partition_tokens, void* workspace,
                     size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (key == nullptr || value == nullptr))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  return decode_impl(desc, out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, scale, partition_tokens, workspace,
                     workspace_bytes, stream);
}

int pa_decode_append_lean(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                          const void* value, void* k_cache, void* v_cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_context_len, float scale, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (num_seqs > 0 && (key == nullptr || value == nullptr))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  return decode_impl(desc, out, q, key, value, k_cache, v_cache, block_tables, max_blocks_per_seq,
                     context_lens, num_seqs, max_context_len, scale, 0, workspace, workspace_bytes, stream,
                     0, true);
}

namespace {
// Arguments of the chunked prefill calls: PA_OK to launch, else the error. A call
// with nothing to do returns PA_OK with *noop set.
int check_prefill_args(const pa_cache_desc* desc, void* out, const void* q, const void* new_k,
                       const void* k_cache, const void* v_cache, const int32_t* query_start_loc,
                       const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                       int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                       float scale, void* stream, bool* noop) {
  *noop = false;
  int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (desc->dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "prefill supports bf16 only");
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || max_seq_len < 0)
    return fail(PA_ERR_INVALID_ARG, "negative size");
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) {
    *noop = true;
    return PA_OK;
  }
  if (!out || !q || !k_cache || !v_cache || !query_start_loc || !seq_lens || !block_tables)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (max_blocks_per_seq <= 0) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be positive");
  if ((int64_t)max_seq_len > (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE)
    return fail(PA_ERR_INVALID_ARG, "max_seq_len exceeds 16 * max_blocks_per_seq");
  if (max_query_len > max_seq_len) return fail(PA_ERR_INVALID_ARG, "max_query_len exceeds max_seq_len");
  if ((int64_t)num_seqs * desc->num_kv_heads > INT32_MAX)
    return fail(PA_ERR_UNSUPPORTED, "num_seqs * num_kv_heads too large");
  if (!std::isfinite(scale)) return fail(PA_ERR_INVALID_ARG, "scale is not finite");
  if (check_mode()) {
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess)
      return fail(PA_ERR_HIP, "stream synchronize failed");
    std::vector<int32_t> qsl, lens, tables;
    if (!fetch(qsl, query_start_loc, (size_t)num_seqs + 1) || !fetch(lens, seq_lens, num_seqs) ||
        !fetch(tables, block_tables, (size_t)num_seqs * max_blocks_per_seq))
      return fail(PA_ERR_HIP, "copy of metadata failed");
    if (qsl[0] != 0 || qsl[num_seqs] != num_tokens)
      return fail(PA_ERR_RANGE, "query_start_loc must start at 0 and end at num_tokens");
    for (int s = 0; s < num_seqs; ++s) {
      const int n = qsl[s + 1] - qsl[s];
      if (n < 0 || n > max_query_len)
        return fail(PA_ERR_RANGE, "chunk of request " + std::to_string(s) + " has " +
                                      std::to_string(n) + " rows");
      if (lens[s] < n || lens[s] > max_seq_len)
        return fail(PA_ERR_RANGE, "seq_lens[" + std::to_string(s) + "] = " +
                                      std::to_string(lens[s]) + " is inconsistent");
    }
    st = check_tables(tables, max_blocks_per_seq, lens, desc->num_blocks);
    if (st != PA_OK) return st;
    if (new_k != nullptr) {  // the chunks' new tokens go to distinct slots
      std::unordered_set<int64_t> seen;
      for (int s = 0; s < num_seqs; ++s)
        for (int i = 0; i < qsl[s + 1] - qsl[s]; ++i) {
          const int pos = lens[s] - (qsl[s + 1] - qsl[s]) + i;
          const int64_t slot = (int64_t)tables[(size_t)s * max_blocks_per_seq + pos / PA_BLOCK_SIZE] *
                                   PA_BLOCK_SIZE + pos % PA_BLOCK_SIZE;
          if (!seen.insert(slot).second)
            return fail(PA_ERR_RANGE, "slot " + std::to_string(slot) + " of request " + std::to_string(s) +
                                          " is written twice");
        }
    }
  }
  return PA_OK;
}

// pa_prefill_chunk; pa_prefill_chunk_append when new_k/new_v are given.
int prefill_impl(const pa_cache_desc* desc, void* out, const void* q, const void* new_k, const void* new_v,
                 const void* k_cache, const void* v_cache, const int32_t* query_start_loc,
                 const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                 float scale, void* stream) {
  bool noop = false;
  const int st = check_prefill_args(desc, out, q, new_k, k_cache, v_cache, query_start_loc, seq_lens, block_tables,
                                    max_blocks_per_seq, num_seqs, num_tokens, max_query_len, max_seq_len, scale,
                                    stream, &noop);
  if (st != PA_OK || noop) return st;
  pa::PrefillArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k_cache;
  a.v = (const uint16_t*)v_cache;
  a.out = (uint16_t*)out;
  a.query_start_loc = query_start_loc;
  a.seq_lens = seq_lens;
  a.block_tables = block_tables;
  a.num_blocks = desc->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.max_query_len = max_query_len;
  a.max_seq_len = max_seq_len;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.scale_log2 = scale * pa::kLog2e;
  a.new_k = (const uint16_t*)new_k;
  a.new_v = (const uint16_t*)new_v;
  return hip_status(pa::launch_prefill(a, desc->head_dim, desc->num_q_heads / desc->num_kv_heads,
                                       as_stream(stream)),
                    "prefill launch");
}
}  // namespace

int pa_prefill_chunk(const pa_cache_desc* desc, void* out, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* query_start_loc, const int32_t* seq_lens,
                     const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                     int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, float scale,
                     void* stream) {
  return prefill_impl(desc, out, q, nullptr, nullptr, k_cache, v_cache, query_start_loc, seq_lens,
                      block_tables, max_blocks_per_seq, num_seqs, num_tokens, max_query_len, max_seq_len,
                      scale, stream);
}

int pa_prefill_chunk_append(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                            const void* value, void* k_cache, void* v_cache, const int32_t* query_start_loc,
                            const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                            int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                            float scale, void* stream) {
  if (num_seqs > 0 && num_tokens > 0 && (key == nullptr || value == nullptr))
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  return prefill_impl(desc, out, q, key, value, k_cache, v_cache, query_start_loc, seq_lens, block_tables,
                      max_blocks_per_seq, num_seqs, num_tokens, max_query_len, max_seq_len, scale, stream);
}

namespace {
// Positions per request pa_prefill_chunk_short takes: the chunk's positions
// times the group fill the 16 columns of the decode's score tile.
int32_t chunk_short_max_rows(const pa_cache_desc* d) { return 16 / (d->num_q_heads / d->num_kv_heads); }
}  // namespace

int32_t pa_prefill_chunk_short_max_query_len(const pa_cache_desc* desc) {
  const int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (desc->dtype != PA_BF16) return fail(PA_ERR_UNSUPPORTED, "prefill supports bf16 only");
  return chunk_short_max_rows(desc);
}

size_t pa_prefill_chunk_short_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                             int32_t max_query_len) {
  if (validate_desc(desc) != PA_OK || desc->dtype != PA_BF16 || num_seqs <= 0 || max_query_len <= 0 ||
      num_seqs > pa::decode_max_balanced_seqs() || max_query_len > chunk_short_max_rows(desc))
    return 0;
  return chunk_short_layout(desc, num_seqs, max_query_len).total;
}

int pa_prefill_chunk_short(const pa_cache_desc* desc, void* out, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                           int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  bool noop = false;
  int st = check_prefill_args(desc, out, q, nullptr, k_cache, v_cache, query_start_loc, seq_lens, block_tables,
                              max_blocks_per_seq, num_seqs, num_tokens, max_query_len, max_seq_len, scale, stream,
                              &noop);
  if (st != PA_OK || noop) return st;
  if (max_query_len > chunk_short_max_rows(desc))
    return fail(PA_ERR_UNSUPPORTED, "max_query_len above " + std::to_string(chunk_short_max_rows(desc)) +
                                        " (16 / q heads per kv head)");
  if (num_seqs > pa::decode_max_balanced_seqs())
    return fail(PA_ERR_UNSUPPORTED, "num_seqs above " + std::to_string(pa::decode_max_balanced_seqs()));
  const DecodeLayout lay = chunk_short_layout(desc, num_seqs, max_query_len);
  if (workspace == nullptr || workspace_bytes < lay.total)
    return fail(PA_ERR_WORKSPACE, "workspace needs " + std::to_string(lay.total) + " bytes");
  pa::DecodeArgs a{};
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.out = out;
  a.block_tables = block_tables;
  a.context_lens = seq_lens;
  a.part_acc = (float*)workspace;
  a.part_ml = (float*)((char*)workspace + lay.acc_bytes);
  a.cum_blocks = (int32_t*)((char*)workspace + lay.acc_bytes + lay.ml_bytes);
  a.split_req = a.cum_blocks + num_seqs + 1;
  a.num_blocks = desc->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.max_context_len = max_seq_len;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.group = desc->num_q_heads / desc->num_kv_heads;
  a.num_workers = lay.workers;
  a.nontemporal = nontemporal_mode(desc, num_seqs, max_seq_len, true);
  a.scale_log2 = scale * pa::kLog2e;
  a.query_start_loc = query_start_loc;
  a.n_cols = max_query_len;
  return hip_status(pa::launch_decode(a, desc->head_dim, true, as_stream(stream)), "short-chunk launch");
}

int pa_copy_blocks(const pa_cache_desc* desc, void* k_cache, void* v_cache,
                   const int32_t* block_pairs, int64_t num_pairs, void* stream) {
  int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs is negative");
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many pairs");
  if (!k_cache || !v_cache || !block_pairs) return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (check_mode()) {
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess)
      return fail(PA_ERR_HIP, "stream synchronize failed");
    std::vector<int32_t> pairs;
    if (!fetch(pairs, block_pairs, (size_t)num_pairs * 2)) return fail(PA_ERR_HIP, "copy of pairs failed");
    std::unordered_set<int32_t> dsts, srcs;
    for (int64_t i = 0; i < num_pairs; ++i) {
      const int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
      if (src < 0 || src >= desc->num_blocks || dst < 0 || dst >= desc->num_blocks)
        return fail(PA_ERR_RANGE, "pair " + std::to_string(i) + " is outside the pool");
      if (!dsts.insert(dst).second)
        return fail(PA_ERR_RANGE, "block " + std::to_string(dst) + " is a destination twice");
      srcs.insert(src);
    }
    for (int32_t d : dsts)
      if (srcs.count(d))
        return fail(PA_ERR_RANGE, "block " + std::to_string(d) + " is both a source and a destination");
  }
  const int64_t block_bytes =
      (int64_t)PA_BLOCK_SIZE * desc->num_kv_heads * desc->head_dim * elem_bytes(desc->dtype);
  return hip_status(pa::launch_copy_blocks(k_cache, v_cache, block_pairs, num_pairs, block_bytes,
                                           desc->num_blocks, as_stream(stream)),
                    "copy_blocks launch");
}

namespace {
// Device-visible address of pinned host memory holding `bytes` bytes at `p`, or
// nullptr if `p` is not such memory (pageable memory would fault on the GPU).
void* host_device_pointer(void* p, size_t bytes) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (attr.type != hipMemoryTypeHost || attr.devicePointer == nullptr) return nullptr;
  void* base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, attr.devicePointer) == hipSuccess && base != nullptr) {
    const size_t off = (size_t)((char*)attr.devicePointer - (char*)base);
    if (off > size || size - off < bytes) return nullptr;  // the buffer is too small
  } else {
    (void)hipGetLastError();
  }
  return attr.devicePointer;
}
}  // namespace

int pa_swap_blocks(const pa_cache_desc* desc, void* k_cache, void* v_cache, void* host_k,
                   void* host_v, int64_t num_host_blocks, const int32_t* block_pairs,
                   int64_t num_pairs, int32_t direction, void* stream) {
  int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (num_pairs < 0) return fail(PA_ERR_INVALID_ARG, "num_pairs is negative");
  if (direction != PA_SWAP_OUT && direction != PA_SWAP_IN)
    return fail(PA_ERR_INVALID_ARG, "direction must be PA_SWAP_OUT or PA_SWAP_IN");
  if (num_host_blocks < 1) return fail(PA_ERR_INVALID_ARG, "num_host_blocks must be >= 1");
  if (num_pairs == 0) return PA_OK;
  if (num_pairs > INT32_MAX) return fail(PA_ERR_UNSUPPORTED, "too many pairs");
  if (!k_cache || !v_cache || !host_k || !host_v || !block_pairs)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  const int64_t block_bytes =
      (int64_t)PA_BLOCK_SIZE * desc->num_kv_heads * desc->head_dim * elem_bytes(desc->dtype);
  void* dk = host_device_pointer(host_k, (size_t)(num_host_blocks * block_bytes));
  void* dv = host_device_pointer(host_v, (size_t)(num_host_blocks * block_bytes));
  if (dk == nullptr || dv == nullptr)
    return fail(PA_ERR_INVALID_ARG, "host_k/host_v must be pinned host memory of num_host_blocks blocks");
  if (check_mode()) {
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess)
      return fail(PA_ERR_HIP, "stream synchronize failed");
    std::vector<int32_t> pairs;
    if (!fetch(pairs, block_pairs, (size_t)num_pairs * 2)) return fail(PA_ERR_HIP, "copy of pairs failed");
    std::unordered_set<int32_t> dsts;
    const bool out = direction == PA_SWAP_OUT;
    for (int64_t i = 0; i < num_pairs; ++i) {
      const int32_t dev = out ? pairs[2 * i] : pairs[2 * i + 1];
      const int32_t hst = out ? pairs[2 * i + 1] : pairs[2 * i];
      if (dev < 0 || dev >= desc->num_blocks || hst < 0 || hst >= num_host_blocks)
        return fail(PA_ERR_RANGE, "pair " + std::to_string(i) + " is outside a pool");
      if (!dsts.insert(pairs[2 * i + 1]).second)
        return fail(PA_ERR_RANGE, "block " + std::to_string(pairs[2 * i + 1]) + " is a destination twice");
    }
  }
  return hip_status(pa::launch_swap_blocks(k_cache, v_cache, dk, dv, block_pairs, num_pairs, block_bytes,
                                           desc->num_blocks, num_host_blocks, direction == PA_SWAP_OUT,
                                           as_stream(stream)),
                    "swap_blocks launch");
}

int pa_gather_kv(const pa_cache_desc* desc, void* dst_k, void* dst_v, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                 void* stream) {
  int st = validate_desc(desc);
  if (st != PA_OK) return st;
  if (num_seqs < 0) return fail(PA_ERR_INVALID_ARG, "num_seqs is negative");
  if (num_seqs == 0 || max_context_len == 0) return PA_OK;
  if (num_seqs > 65535) return fail(PA_ERR_UNSUPPORTED, "num_seqs above 65535");
  if (!dst_k || !dst_v || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PA_ERR_INVALID_ARG, "null pointer argument");
  if (max_context_len < 0 || max_blocks_per_seq <= 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * PA_BLOCK_SIZE)
    return fail(PA_ERR_INVALID_ARG, "max_context_len exceeds 16 * max_blocks_per_seq");
  const int row_bytes = desc->num_kv_heads * desc->head_dim * elem_bytes(desc->dtype);
  return hip_status(pa::launch_gather_kv(dst_k, dst_v, k_cache, v_cache, block_tables,
                                         max_blocks_per_seq, context_lens, num_seqs,
                                         max_context_len, row_bytes, desc->num_kv_heads,
                                         desc->num_blocks, as_stream(stream)),
                    "gather_kv launch");
}

int pa_bench_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes % 16) return fail(PA_ERR_INVALID_ARG, "copy needs 16-byte multiples");
  if (bytes == 0) return PA_OK;
  return hip_status(pa::launch_bench_copy(dst, src, bytes, as_stream(stream)), "copy launch");
}

int pa_bench_read(const void* src, size_t bytes, float* sink, void* stream) {
  if (!src || !sink || bytes % 16) return fail(PA_ERR_INVALID_ARG, "read needs 16-byte multiples");
  if (bytes == 0) return PA_OK;
  return hip_status(pa::launch_bench_read(src, bytes, sink, as_stream(stream)), "read launch");
}

int pa_bench_mfma(const void* operands, int32_t workgroups, int32_t iters, float* sink, void* stream) {
  if (!operands || !sink || workgroups <= 0 || iters < 0)
    return fail(PA_ERR_INVALID_ARG, "mfma needs operands, a sink, workgroups > 0 and iters >= 0");
  return hip_status(pa::launch_bench_mfma(operands, workgroups, iters, sink, as_stream(stream)), "mfma launch");
}

int pa_bench_flush(void* buf, size_t bytes, void* stream) {
  if (!buf || bytes % 16) return fail(PA_ERR_INVALID_ARG, "flush needs 16-byte multiples");
  if (bytes == 0) return PA_OK;
  return hip_status(pa::launch_bench_flush(buf, bytes, as_stream(stream)), "flush launch");
}

}  // extern "C"
