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
 *     Technical Details).
 *   - A preempted request may keep its computed K/V by swapping its blocks out
 *     to a swap space in CPU memory, and swap them in when it resumes (same
 *     page and section; the alternative is recomputation).
 *   - Copies and swaps are queued for the caller as one ordered list of block
 *     operations, run on the device before the step's KV writes.
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
/* The same with a swap space of num_host_blocks (>= 0) blocks in CPU memory, for
 * pa_pool_swap_out / pa_pool_swap_in (pa_pool_create has none). */
pa_block_pool* pa_pool_create_with_swap(int64_t num_blocks, int64_t num_host_blocks,
                                        int32_t prefix_caching);
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
 * of it (queued as a PA_POOL_OP_COPY operation, see pa_pool_take_ops). Returns 0, PA_POOL_NO_SPACE (nothing changed), or
 * an error (computed + hits + num_new_tokens beyond the request's tokens). */
int pa_pool_allocate_slots(pa_block_pool* pool, int64_t req_id, int64_t num_new_tokens,
                           int64_t* hit_tokens);
/* pa_pool_allocate_slots whose blocks also cover num_lookahead positions past the
 * new tokens, which may lie past the request's known tokens: speculative draft
 * tokens that the step writes K/V for and that become tokens only when accepted
 * (the teardown's requests are (computed, known plus speculative) pairs:
 * "Continuous batching: rebuild the batch every step"). Their slots are
 * readable through pa_pool_slot_mapping; pa_pool_commit never counts them until
 * they are appended as tokens. */
int pa_pool_allocate_slots_lookahead(pa_block_pool* pool, int64_t req_id, int64_t num_new_tokens,
                                     int64_t num_lookahead, int64_t* hit_tokens);

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

/* Swap-out (preemption that keeps the K/V instead of recomputing it:
 * aitrending, "The 1960s Operating System Trick That Makes vLLM 4x Faster",
 * Technical Details). The blocks holding the request's computed tokens are
 * paired with free host blocks, in order, and queued as (device, host) pairs;
 * then all its device blocks are released as by pa_pool_free_request. The
 * request keeps its tokens and computed count and is "swapped": it holds no
 * device blocks and cannot be allocated, committed or forked until swapped in.
 * PA_POOL_NO_SPACE (nothing changed) if the swap space is short. A request with
 * nothing computed just releases its blocks and is not swapped. The pairs are
 * queued as PA_POOL_OP_SWAP_OUT operations (see pa_pool_take_ops). */
int pa_pool_swap_out(pa_block_pool* pool, int64_t req_id);
/* Swap-in: one device block per host block, from the head of the free queue as
 * an allocation would take them, queued as PA_POOL_OP_SWAP_IN operations; the
 * request is running again with its computed count, and its host blocks are
 * free again. PA_POOL_NO_SPACE (nothing changed) if the free queue is short. */
int pa_pool_swap_in(pa_block_pool* pool, int64_t req_id);
/* 1 if the request is swapped out, 0 if not, negative if unknown. */
int32_t pa_pool_request_swapped(const pa_block_pool* pool, int64_t req_id);
int64_t pa_pool_num_free_host_blocks(const pa_block_pool* pool);
/* Block operations for the device, in the order the pool performed them:
 * copy-on-write copies (allocate_slots), swap-outs and swap-ins. Moves up to
 * max_ops of them into ops[3 i .. 3 i + 2] = (kind, source, destination),
 * oldest first; returns how many were moved (the rest stay queued).
 *   PA_POOL_OP_COPY      device block -> device block (pa_copy_blocks)
 *   PA_POOL_OP_SWAP_OUT  device block -> host block   (pa_swap_blocks, PA_SWAP_OUT)
 *   PA_POOL_OP_SWAP_IN   host block   -> device block (pa_swap_blocks, PA_SWAP_IN)
 * Run them in this order, all before the KV writes of the step that follows:
 * a block freed by one operation may be handed out again by a later one.
 * Consecutive operations of one kind may run as one call when none of them
 * writes a block that another of them reads or writes. */
#define PA_POOL_OP_COPY 0
#define PA_POOL_OP_SWAP_OUT 1
#define PA_POOL_OP_SWAP_IN 2
int64_t pa_pool_take_ops(pa_block_pool* pool, int32_t* ops, int64_t max_ops);

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
