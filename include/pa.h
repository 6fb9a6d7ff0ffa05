/*
 * pa.h - C ABI of the MI355X (gfx950) paged-KV attention library, libpa.so.
 *
 * The KV cache is one pool of fixed-size blocks of 16 tokens; every request
 * owns a block table mapping its logical token positions to physical blocks,
 * which need not be contiguous and may be shared between requests (arcyou
 * teardown of vLLM paged attention, section "PagedAttention: the KV cache is
 * paged, like virtual memory"; kenhuang vLLM course, "Introduction", section
 * "PagedAttention (intuition)"). Attention is handed the block table and
 * gathers K/V from wherever the blocks live. One scheduler step mixes decode
 * tokens and chunks of long prompts (arcyou teardown, section "Continuous
 * batching: rebuild the batch every step"), so the library offers three
 * calls that one step issues in order on one stream:
 *   pa_write_kv       new tokens' K/V into their slots,
 *   pa_prefill_chunk  causal attention of prompt chunks over cached + new K/V,
 *   pa_decode         one query per request over its whole context.
 *
 * Conventions for every call
 *   - Pointers named k_cache/v_cache/key/value/q/out/workspace and the int32
 *     metadata arrays are DEVICE pointers owned by the caller; every tensor is
 *     dense and row-major in the layout stated below. The library allocates no
 *     device memory and keeps no state between calls.
 *   - Pool layout, K and V alike: [num_blocks][16][num_kv_heads][head_dim].
 *     Token t of a request lives in block block_table[t / 16] at offset t % 16.
 *     A flat slot is block_id * 16 + offset.
 *   - Element type: every tensor of a call (q, K/V pool, new K/V, out) has the
 *     descriptor's dtype: PA_F32 (IEEE float32) or PA_BF16 (bfloat16 bits).
 *     Arithmetic is float32; bf16 outputs are rounded to nearest, ties to even.
 *   - Grouped-query attention: query head h reads kv head h / (Hq / Hkv).
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work; they never synchronise, except in check mode (below).
 *   - Return value: PA_OK or a negative pa_status. Argument errors are found
 *     before anything is enqueued; pa_last_error_detail() then names the
 *     argument. PA_ERR_HIP means the HIP runtime refused a launch.
 *   - Content preconditions (block ids in [0, num_blocks), slots in range and
 *     distinct, lengths within the stated maxima) are checked on the host only
 *     when the environment variable PA_CHECK=1 is set: the call then
 *     synchronises, copies the metadata to the host, and returns PA_ERR_RANGE
 *     on a violation. Without check mode the kernels still never access memory
 *     outside the pool: an out-of-range block id makes the affected outputs NaN,
 *     an out-of-range slot is skipped, and lengths are clamped to the maxima.
 *   - Calls on distinct streams may run concurrently; `out` must not alias an
 *     input; a pa_write_kv must not target a block that another request still
 *     reads (shared blocks are copied before they are written).
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_VERSION 10000 /* major*10000 + minor*100 + patch */
#define PA_BLOCK_SIZE 16

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1, /* null pointer, non-positive size, inconsistent sizes */
  PA_ERR_UNSUPPORTED = -2, /* shape or dtype the library has no kernel for */
  PA_ERR_WORKSPACE = -3,   /* decode workspace missing or too small */
  PA_ERR_RANGE = -4,       /* check mode found metadata outside its range */
  PA_ERR_HIP = -5          /* the HIP runtime reported an error */
} pa_status;

/* One layer's KV pool. Supported: block_size 16; head_dim 64 or 128;
 * num_q_heads a multiple of num_kv_heads with group G = Hq/Hkv; for PA_BF16
 * G must be one of 1, 2, 4, 8, 16; for PA_F32 G <= 16 (decode only). */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t block_size;
  int64_t num_blocks;
  int32_t dtype; /* pa_dtype */
  int32_t reserved; /* must be 0 */
} pa_cache_desc;

/* Write new tokens' K and V into their slots (the "reshape and cache" step).
 * The KV cache grows one token at a time: each new token's K/V rows are
 * stored once, then read by every later token (arcyou teardown, section
 * "The problem both ideas solve"; kenhuang, "PagedAttention (intuition)").
 *   key, value     [num_tokens][Hkv][D]   new tokens, read only
 *   k_cache/v_cache pool tensors, updated in place; only the addressed rows change
 *   slot_mapping   int32 [num_tokens]; slot_mapping[i] = block*16 + offset, or -1
 *                  to skip token i. Slots must be distinct within a call.
 * The copy is bit-exact (no dtype change). num_tokens == 0 is a no-op. */
int pa_write_kv(const pa_cache_desc* desc, const void* key, const void* value,
                void* k_cache, void* v_cache, const int32_t* slot_mapping,
                int64_t num_tokens, void* stream);

/* Keys per split-KV partition that pa_decode chooses when partition_tokens is 0
 * (a multiple of 16), for num_seqs requests of at most max_context_len tokens.
 * The environment variable PA_PARTITION_TOKENS, if set, overrides the choice.
 * Returns a negative pa_status on invalid arguments. */
int32_t pa_decode_partition_tokens(const pa_cache_desc* desc, int32_t num_seqs,
                                   int32_t max_context_len);

/* Bytes of device workspace pa_decode needs for these sizes and this partition
 * size (0 = automatic). 0 means no workspace is needed. Returns 0 for invalid
 * arguments as well; pa_decode reports those. The balanced split's worker
 * count follows the compute units of the calling thread's current device, so
 * the size is for that device: call it with the device of the decode current. */
size_t pa_decode_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                int32_t max_context_len, int32_t partition_tokens);

/* Decode attention: one query per request, at its last position, attending all
 * context_lens[s] tokens of its logical context through its block table
 * (arcyou teardown, section "PagedAttention: the KV cache is paged, like
 * virtual memory": the kernel receives a per-request block table and gathers
 * K/V wherever the blocks live). context_lens[s] counts the request's own
 * newest token, whose K/V must already be written.
 *   out            [num_seqs][Hq][D]  written
 *   q              [num_seqs][Hq][D]
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]; entries at index
 *                  >= ceil(context_lens[s]/16) are never read
 *   context_lens   int32 [num_seqs], 1 <= context_lens[s] <= max_context_len;
 *                  a length <= 0 yields NaN outputs for that request
 *   max_context_len <= 16 * max_blocks_per_seq
 *   scale          multiplies q.k before the softmax (normally 1/sqrt(D))
 *   partition_tokens keys per split-KV partition: 0 = automatic, else a
 *                  positive multiple of 16. A request longer than one partition
 *                  is processed as several partial softmaxes that a second
 *                  kernel merges.
 *   workspace      device scratch of at least pa_decode_workspace_size(...)
 *                  bytes for the same num_seqs, max_context_len and
 *                  partition_tokens; may be NULL when that size is 0. Its
 *                  contents on entry do not matter; concurrent calls need
 *                  separate workspaces.
 * num_seqs == 0 is a no-op. */
int pa_decode(const pa_cache_desc* desc, void* out, const void* q, const void* k_cache,
              const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
              float scale, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
              void* stream);

/* Causal attention for chunks of new tokens (chunked prefill) over the cached
 * tokens plus the chunk itself. A long prompt may be split across steps and a
 * chunk continues after the tokens already computed (arcyou teardown, section
 * "Continuous batching: rebuild the batch every step"); the chunk's K/V must
 * already be written. Row i of request s's chunk of n_s rows sits at absolute
 * position seq_lens[s] - n_s + i and attends keys 0 .. that position.
 * PA_BF16 only.
 *   out, q         [num_tokens][Hq][D]; request s owns rows
 *                  query_start_loc[s] .. query_start_loc[s+1]-1
 *   query_start_loc int32 [num_seqs+1], non-decreasing, query_start_loc[0] = 0,
 *                  query_start_loc[num_seqs] = num_tokens
 *   seq_lens       int32 [num_seqs], total context including the chunk;
 *                  n_s <= seq_lens[s] <= max_seq_len, n_s <= max_query_len
 *   block_tables   int32 [num_seqs][max_blocks_per_seq]
 *   max_seq_len    <= 16 * max_blocks_per_seq
 * Requests with an empty chunk are skipped. num_seqs == 0 is a no-op. */
int pa_prefill_chunk(const pa_cache_desc* desc, void* out, const void* q,
                     const void* k_cache, const void* v_cache, const int32_t* query_start_loc,
                     const int32_t* seq_lens, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, int32_t num_seqs, int32_t num_tokens,
                     int32_t max_query_len, int32_t max_seq_len, float scale, void* stream);

/* Chunked prefill after storing each chunk's new K/V: the same result and pool
 * update as pa_write_kv of every chunk token's K/V into its slot (row i of
 * request s's chunk sits at position seq_lens[s] - n_s + i, in block
 * block_tables[s][position / 16] at offset position % 16) followed by
 * pa_prefill_chunk, in one launch and without the separate write: the kernel
 * reads the chunk's own keys and values from key/value (the cached ones from
 * the pool) and stores the new rows into the pool. With pa_decode_append, a
 * step that mixes prompt chunks and generated tokens (arcyou teardown, section
 * "Continuous batching: rebuild the batch every step") then needs no write
 * launch at all; the KV cache grows one token at a time and every token
 * re-reads all past K/V (arcyou teardown, "The problem both ideas solve").
 * Reading the chunk's rows from key/value is slower than reading them from the
 * pool, so on MI355X this call takes about as long as pa_write_kv followed by
 * pa_prefill_chunk; it saves the launch, not time.
 *   key, value   [num_tokens][Hkv][D] bf16, row t the new token of query row t
 * The blocks covering each chunk's positions must be in its table, distinct
 * between requests and not read by any other request of the call (shared
 * blocks are copied on write first); check mode verifies that the chunks'
 * slots are distinct. All other arguments and the errors are those of
 * pa_prefill_chunk. PA_BF16 only. */
int pa_prefill_chunk_append(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                            const void* value, void* k_cache, void* v_cache, const int32_t* query_start_loc,
                            const int32_t* seq_lens, const int32_t* block_tables, int32_t max_blocks_per_seq,
                            int32_t num_seqs, int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len,
                            float scale, void* stream);

/* pa_prefill_chunk for steps whose chunks are a few tokens long (a request
 * that scores several tokens at once, as speculative decoding does, or the last
 * rows of a prompt): the same result, computed the way pa_decode computes one
 * token. The KV cache of a request is read once per kv head for all its chunk
 * rows (the reads of past K/V dominate such a step: arcyou teardown, "The
 * problem both ideas solve"), split evenly over the device's workgroups by
 * blocks as pa_decode's balanced mode splits them, and a second kernel merges
 * the partial softmaxes of rows whose keys were split. Row i of request s's
 * chunk of n_s rows sits at position seq_lens[s] - n_s + i and attends keys 0 ..
 * that position, as in pa_prefill_chunk; the chunk's K/V must already be in the
 * pool. PA_BF16 only.
 *   max_query_len  at most pa_prefill_chunk_short_max_query_len(desc) =
 *                  16 / (num_q_heads / num_kv_heads): rows times q heads per kv
 *                  head fill at most the 16 columns of the kernel's score tile
 *   num_seqs       at most 8192
 *   workspace      device scratch of at least
 *                  pa_prefill_chunk_short_workspace_size(desc, num_seqs,
 *                  max_query_len) bytes; contents on entry do not matter;
 *                  concurrent calls need separate workspaces
 * All other arguments are those of pa_prefill_chunk. Errors: those of
 * pa_prefill_chunk; PA_ERR_UNSUPPORTED past the limits above; PA_ERR_WORKSPACE
 * for a missing or short workspace. */
int32_t pa_prefill_chunk_short_max_query_len(const pa_cache_desc* desc);
size_t pa_prefill_chunk_short_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                             int32_t max_query_len);
int pa_prefill_chunk_short(const pa_cache_desc* desc, void* out, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* query_start_loc, const int32_t* seq_lens,
                           const int32_t* block_tables, int32_t max_blocks_per_seq, int32_t num_seqs,
                           int32_t num_tokens, int32_t max_query_len, int32_t max_seq_len, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Decode after appending each request's newest token: the same result as
 * pa_write_kv of those tokens into their slots followed by pa_decode. Where the
 * decode runs in its balanced bf16 mode (the default for bf16 pools,
 * partition_tokens == 0) and the requests do not outnumber its workgroups
 * (eight wavefronts per compute unit of the device: 256 workgroups with 8 kv
 * heads on a 256-CU MI355X), no write launch is added: the decode reads the pool up to
 * each newest token, and its merge pass attends that token and stores it.
 * Otherwise the tokens are stored first by a small kernel, then the decode runs. The newest token of
 * request s sits at position context_lens[s] - 1 (context_lens counts it); its
 * slot is read from the request's block table, so the block covering that
 * position must be in the table (and, when shared, already copied on write).
 * The kernel attends the newest key from `key`/`value` and the earlier keys
 * from the pool, and stores the newest K/V into the pool for later steps
 * (the KV cache grows one token at a time and every token re-reads all past
 * K/V: arcyou teardown, "The problem both ideas solve"; kenhuang, "PagedAttention
 * (intuition)").
 *   key, value   [num_seqs][Hkv][D], pool dtype
 * All other arguments, the workspace and the errors are those of pa_decode. */
int pa_decode_append(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                     const void* value, void* k_cache, void* v_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                     int32_t max_context_len, float scale, int32_t partition_tokens, void* workspace,
                     size_t workspace_bytes, void* stream);

/* pa_decode_append for a decode that runs at the same time as other GPU work,
 * typically a pa_prefill_chunk of the same scheduler step on another stream
 * (one step mixes prompt chunks and generated tokens: arcyou teardown, section
 * "Continuous batching: rebuild the batch every step"). Same arguments, result,
 * pool update, workspace (pa_decode_workspace_size with partition_tokens 0) and
 * errors as pa_decode_append with partition_tokens 0. Its kernel keeps each
 * wavefront within 96 registers and one 16-token block in flight, so that one
 * wavefront fits on every SIMD beside a running prefill workgroup and the two
 * calls share the compute units: the decode streams from HBM while the prefill
 * keeps the matrix cores busy. Run alone it streams more slowly than
 * pa_decode_append. bf16 pools with at most 8,192 requests; otherwise it is
 * exactly pa_decode_append. */
int pa_decode_append_lean(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                          const void* value, void* k_cache, void* v_cache, const int32_t* block_tables,
                          int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                          int32_t max_context_len, float scale, void* workspace, size_t workspace_bytes,
                          void* stream);

/* pa_decode_append for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same arguments, result, pool update and errors as pa_decode_append, without
 * the workspace: the split-KV partials go to one fixed device array of
 * PA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every GPU it runs
 * on until the process ends. The call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine); the first call on a device looks up
 * that device's copy of the array once. Sizes whose workspace
 * (pa_decode_workspace_size) exceeds PA_NOALLOC_SCRATCH_BYTES are refused with
 * PA_ERR_WORKSPACE before anything is enqueued; 64 MiB holds, with 32 q heads
 * and head_dim 128 on a 256-CU device, the balanced split of up to 3,776
 * requests of any length. Every call on one GPU shares that GPU's array, and
 * the array keeps the last call's contents (nothing in it needs clearing):
 * calls that overlap on one GPU, e.g. on two streams, race on it and give
 * wrong results. Check mode (PA_CHECK=1) synchronises and copies metadata to
 * the host as for pa_decode_append; leave it off where those are not allowed. */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)
int pa_decode_append_noalloc(const pa_cache_desc* desc, void* out, const void* q, const void* key,
                             const void* value, void* k_cache, void* v_cache, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_context_len, float scale, int32_t partition_tokens, void* stream);

/* Decode when every request shares its first prefix_blocks blocks (the same
 * block ids at the start of every row of block_tables, as when a common prompt
 * is found in the prefix cache): the same result as pa_decode. The prefix is
 * read once for all requests: its attention runs as one dense pass over all the
 * requests' queries on the matrix cores, split into key ranges. Only each
 * request's remaining blocks go through the split-KV decode, and the merge
 * combines both (each key range's and each tail segment's weighted sum of V rows
 * passes to the merge rounded to bf16, its max and sum of exponentials in
 * float32). Sharing full blocks between requests through the prefix cache
 * is arcyou teardown, "PagedAttention: the KV cache is paged, like virtual
 * memory"; the result is attention over each request's whole logical context.
 *   prefix_blocks   0 (then this is pa_decode) or the number of shared blocks;
 *                   every context_lens[s] >= 16 * prefix_blocks
 * bf16 pools, num_seqs <= 8192; other arguments and errors as for pa_decode.
 * PA_CHECK=1 also verifies the lengths and that every row starts with row 0's
 * prefix blocks. The workspace must hold
 * pa_decode_shared_prefix_workspace_size(desc, num_seqs, max_context_len,
 * prefix_blocks) bytes. */
size_t pa_decode_shared_prefix_workspace_size(const pa_cache_desc* desc, int32_t num_seqs,
                                              int32_t max_context_len, int32_t prefix_blocks);
int pa_decode_shared_prefix(const pa_cache_desc* desc, void* out, const void* q, const void* k_cache,
                            const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                            int32_t prefix_blocks, float scale, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Copy whole blocks inside the pool, K and V alike: the copy-on-write step that
 * lets forked sequences share blocks until one of them must write into a shared
 * block, which is then duplicated first (aitrending, "The 1960s Operating System
 * Trick That Makes vLLM 4x Faster", sections TL;DR and Technical Details).
 *   block_pairs  int32 [num_pairs][2]: (source block, destination block)
 * Every destination is distinct and no block is both a source and a destination
 * in one call (check mode verifies this); pairs outside the pool are skipped.
 * The copy is bit-exact. num_pairs == 0 is a no-op. */
int pa_copy_blocks(const pa_cache_desc* desc, void* k_cache, void* v_cache,
                   const int32_t* block_pairs, int64_t num_pairs, void* stream);

/* Move whole blocks (K and V alike) between the device pool and a swap pool in
 * host memory: the swap-out/in that lets a preempted request keep its computed
 * K/V in CPU memory instead of recomputing it (aitrending, "The 1960s Operating
 * System Trick That Makes vLLM 4x Faster", Technical Details: preemption by
 * swapping to CPU memory or by recomputation).
 *   host_k, host_v   [num_host_blocks][16][Hkv][D], same element type as the
 *                    pool, in pinned host memory that the GPU can address
 *                    (hipHostMalloc, or torch pin_memory=True); other memory
 *                    is refused with PA_ERR_INVALID_ARG before any launch.
 *   block_pairs      device int32 [num_pairs][2]:
 *                    direction PA_SWAP_OUT: (device block, host block), device -> host;
 *                    direction PA_SWAP_IN:  (host block, device block), host -> device.
 * Destinations are distinct within a call (check mode verifies this); pairs
 * outside either pool are skipped. The copy is bit-exact. Run a step's swap-out
 * before its swap-in, copy-on-write copies and KV writes: blocks a swap-out
 * frees may be handed out again in the same step. */
#define PA_SWAP_OUT 0
#define PA_SWAP_IN 1
int pa_swap_blocks(const pa_cache_desc* desc, void* k_cache, void* v_cache, void* host_k,
                   void* host_v, int64_t num_host_blocks, const int32_t* block_pairs,
                   int64_t num_pairs, int32_t direction, void* stream);

/* Copy each request's logical K and V out of the pool through its block table,
 * bit for bit, using the same addressing as the attention kernels (an
 * inspection aid for tests).
 *   dst_k, dst_v   [num_seqs][max_context_len][Hkv][D]; rows t >= context_lens[s]
 *                  are left untouched. */
int pa_gather_kv(const pa_cache_desc* desc, void* dst_k, void* dst_v, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                 void* stream);

/* Static text for a status code. */
const char* pa_strerror(int status);
/* Thread-local text naming what the last failing call on this thread rejected. */
const char* pa_last_error_detail(void);
/* PA_VERSION of the built library. */
int pa_version(void);

/* ---- Measurement utilities (not part of attention) ----------------------
 * pa_bench_copy  copies `bytes` (a multiple of 16) from src to dst, 16 B per lane:
 *                a plain streaming kernel of known traffic.
 * pa_bench_read  reads `bytes` (a multiple of 16) from src and writes one word
 *                per workgroup into sink (>= 4096 floats): the read ceiling.
 * pa_bench_flush overwrites `bytes` (a multiple of 16) of buf, e.g. to evict
 *                the last-level cache between timed runs.
 * pa_bench_mfma  `workgroups` workgroups of 512 threads run `iters` rounds of 8
 *                MFMA 32x32x16 bf16 products each (8 * 32768 flop per wavefront and
 *                round) on operand fragments read once from `operands` (device,
 *                at least workgroups * 512 * 128 bytes of bf16 values); each thread
 *                writes one float to sink (workgroups * 512 floats): the dense
 *                matrix-core rate the chip sustains on that data. */
int pa_bench_copy(void* dst, const void* src, size_t bytes, void* stream);
int pa_bench_read(const void* src, size_t bytes, float* sink, void* stream);
int pa_bench_flush(void* buf, size_t bytes, void* stream);
int pa_bench_mfma(const void* operands, int32_t workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
