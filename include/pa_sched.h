/* pa_sched.h - host-side continuous-batching step scheduler (C ABI, CPU only).
 *
 * Builds each step's batch for the device calls of pa.h, following the arcyou
 * teardown of vLLM paged attention, sections "Continuous batching: rebuild the
 * batch every step" and "What happens when the blocks run out":
 *   - A request is only a pair (tokens computed, tokens known); prompts and
 *     generated tokens are the same kind of work. Every step hands out a token
 *     budget: running requests first, in the order they started, each taking
 *     what it still lacks (a long prompt is cut to what the budget has left:
 *     chunked prefill); then waiting requests are admitted in order until the
 *     budget or the free blocks run out. A finished request's blocks are
 *     released at once, so a waiting request can take them in the next step.
 *   - When the pool cannot grow a running request, the scheduler preempts: the
 *     newest running request under first-come-first-served (the lowest
 *     priority, then latest arrival, under priority scheduling). The victim's
 *     blocks are released, its computed count goes back to 0 and it returns to
 *     the head of the waiting queue, to be recomputed; its cached prefix blocks
 *     may still be found in the pool when it is admitted again. With
 *     PA_SCHED_SWAP the victim's computed K/V is swapped out to the pool's host
 *     swap space instead, when it has room, and swapped back in when the request
 *     is admitted again (aitrending, "The 1960s Operating System Trick That
 *     Makes vLLM 4x Faster", Technical Details: swap or recompute).
 *
 * Readings where the pages are silent:
 *   - No waiting request is admitted in a step that preempted.
 *   - Without chunked prefill a waiting request is admitted only if all it
 *     lacks fits the budget left; admission stops at the first that does not.
 *   - Under priority scheduling the waiting queue is ordered by (priority,
 *     arrival), lower value first; a victim already scheduled in the same step
 *     is taken out of the step again.
 *   - A swapped request is admitted only if the free queue covers both its
 *     swap-in and the blocks of the tokens it is given; it resumes at its
 *     computed count. A swap space too small for the victim means recompute.
 *   - When a request's computed count reaches its token count, the step's
 *     sampled token for it is appended; it finishes when it has produced
 *     max_new_tokens tokens (the last one is not appended).
 *   - Speculative tokens (the teardown's request is a pair of computed tokens
 *     and known tokens plus speculative ones, "Continuous batching: rebuild
 *     the batch every step"): draft tokens set for a request hold for the next
 *     step only. A running request whose known tokens all fit the step gets as
 *     many of its drafts as the budget leaves, after its known tokens, and its
 *     blocks cover them; a request still catching up, or not yet running, gets
 *     none. The update takes how many of each request's scheduled drafts were
 *     accepted (a prefix of them): those join the request's tokens as computed,
 *     then the token sampled after them is appended; each counts as a
 *     generated token, up to max_new_tokens. Rejected drafts leave K/V past the
 *     computed count, which later steps overwrite.
 *
 * The step's batch is laid out for one pa_write_kv and one pa_prefill_chunk (the
 * requests given more than one token) and one pa_decode_append (those given
 * one, whose new token is the newest of their context):
 * scheduled requests in batch order are the multi-token ones, the longest
 * first (ties in scheduling order), then the one-token ones in scheduling
 * order; new tokens are packed in the same order. Short chunks (such as a
 * request's drafts) thus end the multi-token group, where a caller can hand
 * them to pa_prefill_chunk_short and the rest to pa_prefill_chunk. The block operations the step caused (swap-outs, swap-ins,
 * copy-on-write copies) are taken from the pool with pa_pool_take_ops and run,
 * in order, before the step's pa_write_kv.
 *
 * Status codes are those of pa_pool.h. Not thread-safe; synchronous.
 */
#ifndef PA_SCHED_H
#define PA_SCHED_H

#include <stdint.h>

#include "pa_pool.h"

#ifdef __cplusplus
extern "C" {
#endif

#define PA_SCHED_FCFS 0
#define PA_SCHED_PRIORITY 1
#define PA_SCHED_RECOMPUTE 0
#define PA_SCHED_SWAP 1

typedef struct {
  int32_t max_num_batched_tokens; /* token budget of one step, >= 1 */
  int32_t max_num_seqs;           /* running requests at most, >= 1 */
  int32_t policy;                 /* PA_SCHED_FCFS or PA_SCHED_PRIORITY */
  int32_t chunked_prefill;        /* 1: a prompt may be split over steps */
  int32_t preempt_mode;           /* PA_SCHED_RECOMPUTE or PA_SCHED_SWAP */
} pa_sched_config;

typedef struct pa_scheduler pa_scheduler;

/* A scheduler over `pool`, which must outlive it and which it alone should
 * change while it lives. NULL on a bad argument. */
pa_scheduler* pa_sched_create(pa_block_pool* pool, const pa_sched_config* config);
void pa_sched_destroy(pa_scheduler* sched);

/* Queue a request (id unused in the pool) with its prompt [num_tokens >= 1];
 * it finishes after max_new_tokens >= 1 generated tokens. arrival order is the
 * order of these calls. */
int pa_sched_add_request(pa_scheduler* sched, int64_t req_id, const int32_t* prompt,
                         int64_t num_tokens, int32_t max_new_tokens, int32_t priority,
                         int64_t cache_salt);

/* Draft tokens [num_drafts >= 0] of a queued request for the next step
 * (replacing any set before); dropped at the next pa_sched_update. */
int pa_sched_set_spec_tokens(pa_scheduler* sched, int64_t req_id, const int32_t* drafts, int32_t num_drafts);
/* The same for num_requests requests at once: request req_ids[i] gets
 * drafts[offsets[i] .. offsets[i+1]-1] (offsets [num_requests + 1], starting at
 * 0, non-decreasing). Checked in full before anything changes. */
int pa_sched_set_spec_tokens_batch(pa_scheduler* sched, int64_t num_requests, const int64_t* req_ids,
                                   const int64_t* offsets, const int32_t* drafts);

/* Plan the next step; returns the number of scheduled requests or an error.
 * The plan stays readable until the next pa_sched_schedule. */
int64_t pa_sched_schedule(pa_scheduler* sched);

/* The plan, in batch order: request id, first new position, new token count. */
int pa_sched_plan(const pa_scheduler* sched, int64_t* req_ids, int32_t* starts, int32_t* counts);
/* Draft tokens scheduled per plan entry: the last drafts[i] of counts[i]. */
int pa_sched_plan_drafts(const pa_scheduler* sched, int32_t* drafts);
int64_t pa_sched_plan_tokens(const pa_scheduler* sched);   /* new tokens in the step */
int64_t pa_sched_plan_prefills(const pa_scheduler* sched); /* leading requests with > 1 token */
int32_t pa_sched_plan_max_blocks(const pa_scheduler* sched); /* widest block table in the step */

/* Device-call metadata of the plan (S scheduled, P of them multi-token, N tokens):
 *   query_start_loc [P + 1]  row offsets of the multi-token requests' tokens
 *   seq_lens [S]             context length after the step (start + count)
 *   block_tables [S * max_blocks] row-major, unused entries set to pad_block
 *   slot_mapping [N]         pool slot of each new token
 *   positions [N]            token position of each new token
 * Any pointer may be NULL to skip that array. max_blocks must be at least
 * pa_sched_plan_max_blocks. */
int pa_sched_batch(const pa_scheduler* sched, int32_t* query_start_loc, int32_t* seq_lens,
                   int32_t* block_tables, int32_t max_blocks, int32_t pad_block,
                   int32_t* slot_mapping, int32_t* positions);

/* After the step has run: record the computed tokens of every scheduled
 * request, append sampled[i] (plan order; read only for requests whose
 * computed count reached their token count), and finish requests that reached
 * max_new_tokens (their blocks are released). Returns the number finished. */
int64_t pa_sched_update(pa_scheduler* sched, const int32_t* sampled);
/* pa_sched_update after a step with draft tokens: num_accepted[i] (plan order,
 * 0 .. drafts[i]) of entry i's scheduled drafts were accepted, and sampled[i]
 * is the token sampled after the last accepted one. NULL num_accepted: none.
 * An out-of-range count is refused before anything changes. */
int64_t pa_sched_update_spec(pa_scheduler* sched, const int32_t* sampled, const int32_t* num_accepted);

int64_t pa_sched_num_waiting(const pa_scheduler* sched);
int64_t pa_sched_num_running(const pa_scheduler* sched);
int64_t pa_sched_num_preemptions(const pa_scheduler* sched); /* since creation */
int64_t pa_sched_num_swaps(const pa_scheduler* sched);       /* preemptions that swapped */
/* Ids of finished requests, oldest first (up to max; removed once taken). */
int64_t pa_sched_take_finished(pa_scheduler* sched, int64_t* ids, int64_t max);
const char* pa_sched_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H */
