/* pa_pool.h - host-side KV block pool with prefix caching (C ABI, CPU only).
 *
 * The pool hands out the physical block ids that the device calls of pa.h read
 * through block tables and write through slot mappings. It follows the paged
 * KV memory described in the arcyou teardown of vLLM paged attention, section
 * "PagedAttention: the KV cache is paged, like virtual memory":
 *   - KV memory is a fixed set of 16-token blocks; a request holds a list of
 *     block ids; growing a request takes enough blocks from a free queue, and
 *     when the free queue cannot cover the growth the call fails and nothing
 *     changes (the caller preempts: same page, "What happens when the blocks run
 *     out").
 *   - Every full block gets a hash chained from its parent block's hash, its 16
 *     token ids and a per-request extra key, so the hash stands for the whole
 *     prefix; a request whose prefix hashes match reuses those blocks by taking
 *     a reference, with no copy.
 *   - A block returns to the free queue when its last reference goes. Blocks
 *     that still hold a cached prefix go to the tail of the queue, so they are
 *     evicted last (LRU); blocks with nothing worth keeping go to the head.
 *     A request's blocks are released last block first, so its prefix survives
 *     longest and a preempted request can get it back on rescheduling.
 *   - Forked requests (parallel sampling) share all blocks; the first write
 *     into a shared, partly filled block makes a private copy (copy-on-write:
 *     aitrending, "The 1960s Operating System Trick That Makes vLLM 4x Faster",
 *     Technical Details). The copies are queued for the caller, who runs them
 *     with pa_copy_blocks before the step's pa_write_kv.
 *
 * Readings where the pages are silent:
 *   - Blocks needed for a request = ceil(tokens it will hold / 16) minus the
 *     blocks it holds (for a new request this is ceil(new tokens / 16)).
 *   - The free queue starts as blocks 0, 1, ..., num_blocks-1 (head first);
 *     allocation pops from the head and drops the popped block's cached hash.
 *   - A prefix hit never covers a request's last token: at least one token is
 *     always computed, so the request produces its next token.
 *   - A lookup hit also checks the block's 16 tokens, extra key and parent hash,
 *     so a 64-bit hash collision between two blocks cannot alias them.
 *   - If a block's hash is already cached in another block (two requests
 *     computed the same prefix at once), the newer block stays uncached.
 *
 * All calls are synchronous, allocate only host memory, and are not
 * thread-safe on one pool. Calls that return a status give PA_POOL_OK, or
 * PA_POOL_NO_SPACE, or a negative error with its detail in pa_pool_last_error;
 * a failing call changes nothing.
 */
#ifndef PA_POOL_H
#define PA_POOL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_POOL_BLOCK_SIZE 16
#define PA_POOL_OK 0
#define PA_POOL_NO_SPACE 1          /* allocate_slots: the free queue is too short */
#define PA_POOL_ERR_INVALID_ARG -1  /* null pointer, bad size, unknown or reused request id */
#define PA_POOL_ERR_RANGE -4        /* a token position or count outside the request */

typedef struct pa_block_pool pa_block_pool;

/* A pool of num_blocks (>= 1) blocks. prefix_caching: 0 off, 1 on.
 * Returns NULL on a bad argument or when host memory runs out. */
pa_block_pool* pa_pool_create(int64_t num_blocks, int32_t prefix_caching);
void pa_pool_destroy(pa_block_pool* pool);

/* Register request req_id (unused id, >= 0) with its prompt tokens [num_tokens >= 1].
 * cache_salt is the extra key mixed into every block hash (e.g. an adapter id):
 * requests with different salts never share blocks. The pool copies tokens. */
int pa_pool_add_request(pa_block_pool* pool, int64_t req_id, const int32_t* tokens,
                        int64_t num_tokens, int64_t cache_salt);

/* Append n >= 0 tokens (generated ones) to a request's token list. */
int pa_pool_append_tokens(pa_block_pool* pool, int64_t req_id, const int32_t* tokens, int64_t n);

/* Query only: how many tokens a prefix-cache hit would give this request now
 * (a multiple of 16, 0 unless it holds no blocks). Negative on error. */
int64_t pa_pool_prefix_hit_tokens(const pa_block_pool* pool, int64_t req_id);

/* Make the request's blocks cover num_computed + hits + num_new_tokens tokens.
 * A request that holds no blocks first takes the prefix-cache hit (exactly what
 * pa_pool_prefix_hit_tokens reports), which advances its computed count; the
 * hit token count goes to *hit_tokens (may be NULL). If the block that the new
 * tokens start in is partly filled and shared, the request gets a private copy
 * of it (queued, see pa_pool_take_copies). Returns 0, PA_POOL_NO_SPACE (nothing changed), or
 * an error (computed + hits + num_new_tokens beyond the request's tokens). */
int pa_pool_allocate_slots(pa_block_pool* pool, int64_t req_id, int64_t num_new_tokens,
                           int64_t* hit_tokens);

/* Record that the first num_computed tokens now hold K/V in the pool (never
 * decreasing, at most the tokens the blocks cover). Every block that became
 * full is hashed and, with prefix caching, entered in the cache. */
int pa_pool_commit(pa_block_pool* pool, int64_t req_id, int64_t num_computed);

/* Release the request's blocks, last block first. keep_request = 0: forget the
 * request (finished). keep_request = 1: preemption; the request keeps its
 * tokens with a computed count of 0 and may be scheduled again. */
int pa_pool_free_request(pa_block_pool* pool, int64_t req_id, int32_t keep_request);

/* New request child_id with parent_id's tokens, computed count and cache salt,
 * sharing the blocks that hold the computed tokens (one more reference each). */
int pa_pool_fork(pa_block_pool* pool, int64_t parent_id, int64_t child_id);

/* Move up to max_pairs pending copy-on-write pairs (source block, destination
 * block) into pairs[2*i], pairs[2*i+1], oldest first; returns how many were
 * moved (the rest stay queued). */
int64_t pa_pool_take_copies(pa_block_pool* pool, int32_t* pairs, int64_t max_pairs);

/* Queries. Request queries return a negative status for an unknown request. */
int64_t pa_pool_num_blocks(const pa_block_pool* pool);
int64_t pa_pool_num_free_blocks(const pa_block_pool* pool);   /* length of the free queue */
int64_t pa_pool_num_cached_blocks(const pa_block_pool* pool); /* blocks holding a cached hash */
int32_t pa_pool_ref_count(const pa_block_pool* pool, int32_t block); /* -1 if out of range */
int64_t pa_pool_request_tokens(const pa_block_pool* pool, int64_t req_id);
int64_t pa_pool_request_computed(const pa_block_pool* pool, int64_t req_id);
/* Copies up to max ids of the request's block table to out; returns its length. */
int64_t pa_pool_block_table(const pa_block_pool* pool, int64_t req_id, int32_t* out, int64_t max);
/* Slots (block * 16 + offset) of token positions start .. start + n - 1, which
 * must lie inside the request's blocks. */
int pa_pool_slot_mapping(const pa_block_pool* pool, int64_t req_id, int64_t start, int64_t n,
                         int32_t* out);
/* The free queue, head first (up to max ids); returns its length. */
int64_t pa_pool_free_queue(const pa_block_pool* pool, int32_t* out, int64_t max);
/* Chained hash of a request's full block i (0-based), for inspection; 0 if the
 * block is not full. */
uint64_t pa_pool_block_hash(const pa_block_pool* pool, int64_t req_id, int64_t i);
/* Thread-local text naming what the last failing call rejected. */
const char* pa_pool_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_POOL_H */
