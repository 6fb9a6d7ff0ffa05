// block_pool.cpp - host-side KV block pool with prefix caching (see pa_pool.h).
//
// Paged KV memory as in the arcyou teardown of vLLM paged attention, section
// "PagedAttention: the KV cache is paged, like virtual memory": fixed 16-token
// blocks, a free queue, per-request block lists, full blocks hashed by chaining
// the parent's hash with the block's tokens and an extra key, reference counts
// for shared prefixes, cached free blocks kept at the tail of the free queue
// (evicted last) and a request's blocks released last block first. Forked
// requests share blocks until one writes into a shared, partly filled block,
// which is then copied; a preempted request may keep its K/V by swapping its
// blocks to a host swap space (aitrending, "The 1960s Operating System Trick
// That Makes vLLM 4x Faster", Technical Details). Copies and swaps are queued
// as one ordered list of block operations for the device.
//
// The free queue is an intrusive doubly linked list over block ids, so taking a
// cached free block out of the middle on a prefix hit is O(1). The prefix cache
// maps a 64-bit chained hash to a block; a hit is accepted only when the block's
// own record (its tokens, extra key and parent hash) matches, so a hash
// collision can only cost a miss, never alias two prefixes.
#include "pa_pool.h"

#include <algorithm>
#include <array>
#include <cstring>
#include <deque>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

namespace {

constexpr int kB = PA_POOL_BLOCK_SIZE;
constexpr uint64_t kRootHash = 0x243f6a8885a308d3ull;  // parent hash of a request's first block

thread_local std::string g_error;

int fail(int status, const std::string& what) {
  g_error = what;
  return status;
}

// splitmix64 finalizer (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014): a bijective 64-bit mix.
uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

// Hash of one full block: chained from its parent's hash, then the extra key,
// then the 16 token ids in order.
uint64_t block_hash(uint64_t parent, int64_t salt, const int32_t* tokens) {
  uint64_t h = mix64(parent ^ 0x9e3779b97f4a7c15ull);
  h = mix64(h ^ (uint64_t)salt);
  for (int i = 0; i < kB; ++i) h = mix64(h ^ ((uint64_t)(uint32_t)tokens[i] + 0x9e3779b97f4a7c15ull * (i + 1)));
  return h;
}

struct Block {
  int32_t ref = 0;
  int32_t prev = -1, next = -1;  // free-queue links
  bool in_free = false;
  bool cached = false;           // holds the prefix-cache entry `hash`
  uint64_t hash = 0, parent_hash = 0;
  int64_t salt = 0;
  std::array<int32_t, kB> tokens{};
};

struct Request {
  std::vector<int32_t> tokens;
  int64_t salt = 0;
  int64_t computed = 0;
  int64_t hashed = 0;               // full blocks already offered to the cache
  std::vector<int32_t> blocks;
  bool swapped = false;             // computed K/V lives in host_blocks
  std::vector<int32_t> host_blocks;
  mutable std::vector<uint64_t> hashes;  // chained hashes of full blocks, grown on demand

  int64_t full_blocks() const { return (int64_t)tokens.size() / kB; }
  uint64_t hash_of(int64_t i) const {  // i < full_blocks()
    while ((int64_t)hashes.size() <= i) {
      const int64_t j = (int64_t)hashes.size();
      hashes.push_back(block_hash(j ? hashes[j - 1] : kRootHash, salt, &tokens[j * kB]));
    }
    return hashes[i];
  }
  uint64_t parent_of(int64_t i) const { return i ? hash_of(i - 1) : kRootHash; }
};

}  // namespace

struct pa_block_pool {
  std::vector<Block> blocks;
  int32_t head = -1, tail = -1;
  int64_t nfree = 0, ncached = 0;
  bool prefix = false;
  std::unordered_map<uint64_t, int32_t> cache;
  std::unordered_map<int64_t, Request> reqs;
  // block operations for the device, in the order the pool performed them
  struct Op {
    int32_t kind, src, dst;
  };
  std::deque<Op> ops;
  int64_t num_host = 0;
  std::deque<int32_t> host_free;  // swap space, head first

  void unlink(int32_t id) {
    Block& b = blocks[id];
    if (b.prev >= 0) blocks[b.prev].next = b.next; else head = b.next;
    if (b.next >= 0) blocks[b.next].prev = b.prev; else tail = b.prev;
    b.prev = b.next = -1;
    b.in_free = false;
    --nfree;
  }
  void push_tail(int32_t id) {
    Block& b = blocks[id];
    b.prev = tail;
    b.next = -1;
    if (tail >= 0) blocks[tail].next = id; else head = id;
    tail = id;
    b.in_free = true;
    ++nfree;
  }
  void push_head(int32_t id) {
    Block& b = blocks[id];
    b.next = head;
    b.prev = -1;
    if (head >= 0) blocks[head].prev = id; else tail = id;
    head = id;
    b.in_free = true;
    ++nfree;
  }
  void uncache(int32_t id) {
    Block& b = blocks[id];
    if (!b.cached) return;
    auto it = cache.find(b.hash);
    if (it != cache.end() && it->second == id) cache.erase(it);
    b.cached = false;
    --ncached;
  }
  // Pop the head of the free queue for reuse: its cached prefix (if any) is evicted.
  int32_t pop_head() {
    const int32_t id = head;
    unlink(id);
    uncache(id);
    blocks[id].ref = 1;
    return id;
  }
  void release(int32_t id) {
    Block& b = blocks[id];
    if (--b.ref == 0) {
      if (b.cached) push_tail(id); else push_head(id);
    }
  }
  // Cached block holding exactly full block i of request r, or -1.
  int32_t lookup(const Request& r, int64_t i) const {
    const uint64_t h = r.hash_of(i);
    auto it = cache.find(h);
    if (it == cache.end()) return -1;
    const Block& b = blocks[it->second];
    if (!b.cached || b.hash != h || b.parent_hash != r.parent_of(i) || b.salt != r.salt ||
        std::memcmp(b.tokens.data(), &r.tokens[i * kB], sizeof(int32_t) * kB) != 0)
      return -1;
    return it->second;
  }
  // Blocks a prefix hit would give request r now (leaving its last token to compute).
  std::vector<int32_t> prefix_hits(const Request& r) const {
    std::vector<int32_t> hits;
    if (!prefix || !r.blocks.empty() || r.swapped) return hits;
    const int64_t max_blocks = ((int64_t)r.tokens.size() - 1) / kB;
    for (int64_t i = 0; i < max_blocks; ++i) {
      const int32_t id = lookup(r, i);
      if (id < 0) break;
      hits.push_back(id);
    }
    return hits;
  }
  Request* find(int64_t id) {
    auto it = reqs.find(id);
    return it == reqs.end() ? nullptr : &it->second;
  }
  const Request* find(int64_t id) const {
    auto it = reqs.find(id);
    return it == reqs.end() ? nullptr : &it->second;
  }
};

namespace {
int unknown(int64_t id) { return fail(PA_POOL_ERR_INVALID_ARG, "unknown request " + std::to_string(id)); }
}  // namespace

extern "C" {

pa_block_pool* pa_pool_create(int64_t num_blocks, int32_t prefix_caching) {
  return pa_pool_create_with_swap(num_blocks, 0, prefix_caching);
}

pa_block_pool* pa_pool_create_with_swap(int64_t num_blocks, int64_t num_host_blocks,
                                        int32_t prefix_caching) {
  if (num_blocks < 1 || num_blocks > INT32_MAX / kB || num_host_blocks < 0 ||
      num_host_blocks > INT32_MAX / kB) {
    fail(PA_POOL_ERR_INVALID_ARG, "num_blocks must be in [1, 2^31 / 16), num_host_blocks in [0, 2^31 / 16)");
    return nullptr;
  }
  pa_block_pool* p = new (std::nothrow) pa_block_pool;
  if (p == nullptr) return nullptr;
  try {
    p->blocks.resize((size_t)num_blocks);
  } catch (...) {
    delete p;
    fail(PA_POOL_ERR_INVALID_ARG, "out of host memory");
    return nullptr;
  }
  p->prefix = prefix_caching != 0;
  for (int32_t i = 0; i < (int32_t)num_blocks; ++i) p->push_tail(i);
  p->num_host = num_host_blocks;
  for (int32_t i = 0; i < (int32_t)num_host_blocks; ++i) p->host_free.push_back(i);
  return p;
}

void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

int pa_pool_add_request(pa_block_pool* pool, int64_t req_id, const int32_t* tokens,
                        int64_t num_tokens, int64_t cache_salt) {
  if (pool == nullptr || tokens == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  if (req_id < 0) return fail(PA_POOL_ERR_INVALID_ARG, "request ids are >= 0");
  if (num_tokens < 1) return fail(PA_POOL_ERR_INVALID_ARG, "a request needs at least one token");
  if (pool->reqs.count(req_id)) return fail(PA_POOL_ERR_INVALID_ARG, "request id in use");
  Request& r = pool->reqs[req_id];
  r.tokens.assign(tokens, tokens + num_tokens);
  r.salt = cache_salt;
  return PA_POOL_OK;
}

int pa_pool_append_tokens(pa_block_pool* pool, int64_t req_id, const int32_t* tokens, int64_t n) {
  if (pool == nullptr || (n > 0 && tokens == nullptr)) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  if (n < 0) return fail(PA_POOL_ERR_INVALID_ARG, "negative token count");
  Request* r = pool->find(req_id);
  if (r == nullptr) return unknown(req_id);
  r->tokens.insert(r->tokens.end(), tokens, tokens + n);
  return PA_POOL_OK;
}

int64_t pa_pool_prefix_hit_tokens(const pa_block_pool* pool, int64_t req_id) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  const Request* r = pool->find(req_id);
  if (r == nullptr) return unknown(req_id);
  return (int64_t)pool->prefix_hits(*r).size() * kB;
}

int pa_pool_allocate_slots(pa_block_pool* pool, int64_t req_id, int64_t num_new_tokens,
                           int64_t* hit_tokens) {
  return pa_pool_allocate_slots_lookahead(pool, req_id, num_new_tokens, 0, hit_tokens);
}

int pa_pool_allocate_slots_lookahead(pa_block_pool* pool, int64_t req_id, int64_t num_new_tokens,
                                     int64_t num_lookahead, int64_t* hit_tokens) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  if (num_new_tokens < 0 || num_lookahead < 0) return fail(PA_POOL_ERR_INVALID_ARG, "negative token count");
  Request* rp = pool->find(req_id);
  if (rp == nullptr) return unknown(req_id);
  Request& r = *rp;
  if (r.swapped) return fail(PA_POOL_ERR_INVALID_ARG, "request is swapped out: swap it in first");
  const std::vector<int32_t> hits = pool->prefix_hits(r);
  const int64_t start = r.computed + (int64_t)hits.size() * kB;  // first token written
  const int64_t total = start + num_new_tokens;
  if (total > (int64_t)r.tokens.size())
    return fail(PA_POOL_ERR_RANGE, "allocation beyond the request's tokens");
  const int64_t held = (int64_t)r.blocks.size() + (int64_t)hits.size();
  const int64_t fresh = std::max<int64_t>(0, (total + num_lookahead + kB - 1) / kB - held);
  // copy-on-write: new tokens start inside a partly filled block that others share
  const int64_t first = start / kB;
  const bool cow = num_new_tokens + num_lookahead > 0 && start % kB != 0 && first < (int64_t)r.blocks.size() &&
                   pool->blocks[r.blocks[first]].ref > 1;
  int64_t from_queue = fresh + (cow ? 1 : 0);
  for (int32_t id : hits)
    if (pool->blocks[id].ref == 0) ++from_queue;  // a cached free block leaves the queue
  if (from_queue > pool->nfree) return PA_POOL_NO_SPACE;

  for (int32_t id : hits) {
    Block& b = pool->blocks[id];
    if (b.ref == 0) pool->unlink(id);
    ++b.ref;
    r.blocks.push_back(id);
  }
  r.computed = start;
  if (!hits.empty()) r.hashed = (int64_t)hits.size();  // hit blocks are cached already
  if (cow) {
    const int32_t src = r.blocks[first];
    const int32_t dst = pool->pop_head();
    --pool->blocks[src].ref;  // was > 1
    r.blocks[first] = dst;
    pool->ops.push_back({PA_POOL_OP_COPY, src, dst});
  }
  for (int64_t i = 0; i < fresh; ++i) r.blocks.push_back(pool->pop_head());
  if (hit_tokens != nullptr) *hit_tokens = (int64_t)hits.size() * kB;
  return PA_POOL_OK;
}

int pa_pool_commit(pa_block_pool* pool, int64_t req_id, int64_t num_computed) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  Request* rp = pool->find(req_id);
  if (rp == nullptr) return unknown(req_id);
  Request& r = *rp;
  const int64_t cover = std::min<int64_t>((int64_t)r.blocks.size() * kB, (int64_t)r.tokens.size());
  if (num_computed < r.computed || num_computed > cover)
    return fail(PA_POOL_ERR_RANGE, "computed count must grow and stay inside the request's blocks");
  r.computed = num_computed;
  const int64_t full = num_computed / kB;
  for (int64_t i = r.hashed; i < full; ++i) {
    if (!pool->prefix) break;
    const int32_t id = r.blocks[i];
    Block& b = pool->blocks[id];
    if (b.cached) continue;
    const uint64_t h = r.hash_of(i);
    if (pool->cache.count(h)) continue;  // the same prefix is cached in another block
    b.cached = true;
    b.hash = h;
    b.parent_hash = r.parent_of(i);
    b.salt = r.salt;
    std::memcpy(b.tokens.data(), &r.tokens[i * kB], sizeof(int32_t) * kB);
    pool->cache.emplace(h, id);
    ++pool->ncached;
  }
  r.hashed = std::max(r.hashed, full);
  return PA_POOL_OK;
}

int pa_pool_free_request(pa_block_pool* pool, int64_t req_id, int32_t keep_request) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  Request* rp = pool->find(req_id);
  if (rp == nullptr) return unknown(req_id);
  for (auto it = rp->blocks.rbegin(); it != rp->blocks.rend(); ++it) pool->release(*it);
  for (int32_t h : rp->host_blocks) pool->host_free.push_back(h);
  if (keep_request) {
    rp->blocks.clear();
    rp->host_blocks.clear();
    rp->swapped = false;
    rp->computed = 0;
    rp->hashed = 0;
  } else {
    pool->reqs.erase(req_id);
  }
  return PA_POOL_OK;
}

int pa_pool_fork(pa_block_pool* pool, int64_t parent_id, int64_t child_id) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  if (child_id < 0) return fail(PA_POOL_ERR_INVALID_ARG, "request ids are >= 0");
  if (pool->reqs.count(child_id)) return fail(PA_POOL_ERR_INVALID_ARG, "request id in use");
  const Request* pp = pool->find(parent_id);
  if (pp == nullptr) return unknown(parent_id);
  if (pp->swapped) return fail(PA_POOL_ERR_INVALID_ARG, "parent is swapped out");
  Request child;
  child.tokens = pp->tokens;
  child.salt = pp->salt;
  child.computed = pp->computed;
  child.hashed = std::min(pp->hashed, pp->computed / kB);
  child.hashes = pp->hashes;
  const int64_t share = (pp->computed + kB - 1) / kB;
  child.blocks.assign(pp->blocks.begin(), pp->blocks.begin() + share);
  for (int32_t id : child.blocks) ++pool->blocks[id].ref;
  pool->reqs.emplace(child_id, std::move(child));
  return PA_POOL_OK;
}

int pa_pool_swap_out(pa_block_pool* pool, int64_t req_id) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  Request* rp = pool->find(req_id);
  if (rp == nullptr) return unknown(req_id);
  Request& r = *rp;
  if (r.swapped) return fail(PA_POOL_ERR_INVALID_ARG, "request is already swapped out");
  const int64_t keep = (r.computed + kB - 1) / kB;  // blocks holding computed tokens
  if (keep > (int64_t)pool->host_free.size()) return PA_POOL_NO_SPACE;
  for (int64_t i = 0; i < keep; ++i) {
    const int32_t h = pool->host_free.front();
    pool->host_free.pop_front();
    pool->ops.push_back({PA_POOL_OP_SWAP_OUT, r.blocks[i], h});
    r.host_blocks.push_back(h);
  }
  for (auto it = r.blocks.rbegin(); it != r.blocks.rend(); ++it) pool->release(*it);
  r.blocks.clear();
  r.hashed = 0;
  r.swapped = keep > 0;
  return PA_POOL_OK;
}

int pa_pool_swap_in(pa_block_pool* pool, int64_t req_id) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  Request* rp = pool->find(req_id);
  if (rp == nullptr) return unknown(req_id);
  Request& r = *rp;
  if (!r.swapped) return fail(PA_POOL_ERR_INVALID_ARG, "request is not swapped out");
  if ((int64_t)r.host_blocks.size() > pool->nfree) return PA_POOL_NO_SPACE;
  for (int32_t h : r.host_blocks) {
    const int32_t d = pool->pop_head();
    pool->ops.push_back({PA_POOL_OP_SWAP_IN, h, d});
    r.blocks.push_back(d);
    pool->host_free.push_back(h);  // its copy-out precedes any later reuse in the op order
  }
  r.host_blocks.clear();
  r.swapped = false;
  r.hashed = 0;  // the next commit offers these full blocks to the prefix cache again
  return PA_POOL_OK;
}

int32_t pa_pool_request_swapped(const pa_block_pool* pool, int64_t req_id) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  const Request* r = pool->find(req_id);
  return r ? (int32_t)r->swapped : unknown(req_id);
}

int64_t pa_pool_num_free_host_blocks(const pa_block_pool* pool) {
  return pool ? (int64_t)pool->host_free.size() : fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
}

int64_t pa_pool_take_ops(pa_block_pool* pool, int32_t* ops, int64_t max_ops) {
  if (pool == nullptr || (max_ops > 0 && ops == nullptr)) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  int64_t n = 0;
  while (n < max_ops && !pool->ops.empty()) {
    const pa_block_pool::Op& o = pool->ops.front();
    ops[3 * n] = o.kind;
    ops[3 * n + 1] = o.src;
    ops[3 * n + 2] = o.dst;
    pool->ops.pop_front();
    ++n;
  }
  return n;
}

int64_t pa_pool_num_blocks(const pa_block_pool* pool) {
  return pool ? (int64_t)pool->blocks.size() : fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
}
int64_t pa_pool_num_free_blocks(const pa_block_pool* pool) {
  return pool ? pool->nfree : fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
}
int64_t pa_pool_num_cached_blocks(const pa_block_pool* pool) {
  return pool ? pool->ncached : fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
}
int32_t pa_pool_ref_count(const pa_block_pool* pool, int32_t block) {
  if (pool == nullptr || block < 0 || block >= (int32_t)pool->blocks.size()) return -1;
  return pool->blocks[block].ref;
}
int64_t pa_pool_request_tokens(const pa_block_pool* pool, int64_t req_id) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  const Request* r = pool->find(req_id);
  return r ? (int64_t)r->tokens.size() : unknown(req_id);
}
int64_t pa_pool_request_computed(const pa_block_pool* pool, int64_t req_id) {
  if (pool == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  const Request* r = pool->find(req_id);
  return r ? r->computed : unknown(req_id);
}
int64_t pa_pool_block_table(const pa_block_pool* pool, int64_t req_id, int32_t* out, int64_t max) {
  if (pool == nullptr || (max > 0 && out == nullptr)) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  const Request* r = pool->find(req_id);
  if (r == nullptr) return unknown(req_id);
  const int64_t n = (int64_t)r->blocks.size();
  for (int64_t i = 0; i < std::min(n, max); ++i) out[i] = r->blocks[i];
  return n;
}
int pa_pool_slot_mapping(const pa_block_pool* pool, int64_t req_id, int64_t start, int64_t n,
                         int32_t* out) {
  if (pool == nullptr || (n > 0 && out == nullptr)) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  const Request* r = pool->find(req_id);
  if (r == nullptr) return unknown(req_id);
  if (start < 0 || n < 0 || start + n > (int64_t)r->blocks.size() * kB)
    return fail(PA_POOL_ERR_RANGE, "positions outside the request's blocks");
  for (int64_t i = 0; i < n; ++i) {
    const int64_t pos = start + i;
    out[i] = r->blocks[pos / kB] * kB + (int32_t)(pos % kB);
  }
  return PA_POOL_OK;
}
int64_t pa_pool_free_queue(const pa_block_pool* pool, int32_t* out, int64_t max) {
  if (pool == nullptr || (max > 0 && out == nullptr)) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  int64_t n = 0;
  for (int32_t id = pool->head; id >= 0; id = pool->blocks[id].next, ++n)
    if (n < max) out[n] = id;
  return n;
}
uint64_t pa_pool_block_hash(const pa_block_pool* pool, int64_t req_id, int64_t i) {
  if (pool == nullptr) return 0;
  const Request* r = pool->find(req_id);
  if (r == nullptr || i < 0 || i >= r->full_blocks()) return 0;
  return r->hash_of(i);
}
const char* pa_pool_last_error(void) { return g_error.c_str(); }

}  // extern "C"
