// sched.cpp - continuous-batching step scheduler over the host block pool (see pa_sched.h).
//
// One step (arcyou teardown of vLLM paged attention, "Continuous batching:
// rebuild the batch every step" and "What happens when the blocks run out"):
// running requests first, in start order, each given what it lacks up to the
// budget left; a request the pool cannot grow triggers preemption of the newest
// running request (FCFS) or of the lowest-priority, latest-arrival one
// (priority), which returns to the waiting queue with nothing computed, or,
// in swap mode, with its computed K/V swapped out to host memory; then, unless
// the step preempted, waiting requests are admitted in queue order. A running
// request may also carry draft tokens for one step (speculative decoding): the
// teardown's request is a (computed, known plus speculative) pair.
#include "pa_sched.h"

#include <algorithm>
#include <deque>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

namespace {

thread_local std::string g_error;

int fail(int status, const std::string& what) {
  g_error = what;
  return status;
}

struct SchedRequest {
  int32_t max_new = 1;
  int32_t priority = 0;
  int64_t arrival = 0;
  int32_t produced = 0;
};

struct Item {
  int64_t id;
  int32_t start, count;
  int32_t drafts;  // the last `drafts` positions of count are draft tokens
};

}  // namespace

struct pa_scheduler {
  pa_block_pool* pool = nullptr;
  pa_sched_config cfg{};
  std::unordered_map<int64_t, SchedRequest> reqs;
  std::deque<int64_t> waiting;   // head first
  std::vector<int64_t> running;  // start order
  std::vector<Item> plan;        // batch order
  std::unordered_map<int64_t, std::vector<int32_t>> drafts;  // for the next step
  std::deque<int64_t> finished;
  int64_t preemptions = 0;
  int64_t swaps = 0;
  int64_t arrivals = 0;

  bool before(int64_t a, int64_t b) const {  // waiting order under priority scheduling
    const SchedRequest& x = reqs.at(a);
    const SchedRequest& y = reqs.at(b);
    return x.priority != y.priority ? x.priority < y.priority : x.arrival < y.arrival;
  }
  void enqueue_waiting(int64_t id, bool preempted) {
    if (cfg.policy == PA_SCHED_PRIORITY) {
      auto it = std::find_if(waiting.begin(), waiting.end(), [&](int64_t w) { return before(id, w); });
      waiting.insert(it, id);
    } else if (preempted) {
      waiting.push_front(id);
    } else {
      waiting.push_back(id);
    }
  }
  size_t victim_index() const {
    if (cfg.policy != PA_SCHED_PRIORITY) return running.size() - 1;
    size_t v = 0;
    for (size_t i = 1; i < running.size(); ++i) {
      const SchedRequest& a = reqs.at(running[i]);
      const SchedRequest& b = reqs.at(running[v]);
      if (a.priority > b.priority || (a.priority == b.priority && a.arrival > b.arrival)) v = i;
    }
    return v;
  }
};

extern "C" {

pa_scheduler* pa_sched_create(pa_block_pool* pool, const pa_sched_config* config) {
  if (pool == nullptr || config == nullptr || config->max_num_batched_tokens < 1 ||
      config->max_num_seqs < 1 ||
      (config->policy != PA_SCHED_FCFS && config->policy != PA_SCHED_PRIORITY) ||
      (config->preempt_mode != PA_SCHED_RECOMPUTE && config->preempt_mode != PA_SCHED_SWAP)) {
    fail(PA_POOL_ERR_INVALID_ARG, "bad pool or configuration");
    return nullptr;
  }
  pa_scheduler* s = new (std::nothrow) pa_scheduler;
  if (s == nullptr) return nullptr;
  s->pool = pool;
  s->cfg = *config;
  return s;
}

void pa_sched_destroy(pa_scheduler* sched) { delete sched; }

int pa_sched_add_request(pa_scheduler* s, int64_t req_id, const int32_t* prompt, int64_t num_tokens,
                         int32_t max_new_tokens, int32_t priority, int64_t cache_salt) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  if (max_new_tokens < 1) return fail(PA_POOL_ERR_INVALID_ARG, "max_new_tokens must be >= 1");
  const int st = pa_pool_add_request(s->pool, req_id, prompt, num_tokens, cache_salt);
  if (st != PA_POOL_OK) return fail(st, pa_pool_last_error());
  SchedRequest r;
  r.max_new = max_new_tokens;
  r.priority = priority;
  r.arrival = s->arrivals++;
  s->reqs[req_id] = r;
  s->enqueue_waiting(req_id, false);
  return PA_POOL_OK;
}

int pa_sched_set_spec_tokens(pa_scheduler* s, int64_t req_id, const int32_t* drafts, int32_t num_drafts) {
  if (s == nullptr || num_drafts < 0 || (num_drafts > 0 && drafts == nullptr))
    return fail(PA_POOL_ERR_INVALID_ARG, "bad draft tokens");
  if (s->reqs.count(req_id) == 0) return fail(PA_POOL_ERR_INVALID_ARG, "unknown request");
  s->drafts[req_id].assign(drafts, drafts + num_drafts);
  return PA_POOL_OK;
}

int pa_sched_set_spec_tokens_batch(pa_scheduler* s, int64_t num_requests, const int64_t* req_ids,
                                   const int64_t* offsets, const int32_t* drafts) {
  if (s == nullptr || num_requests < 0 || (num_requests > 0 && (req_ids == nullptr || offsets == nullptr)))
    return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  for (int64_t i = 0; i < num_requests; ++i) {  // check everything before changing anything
    if (s->reqs.count(req_ids[i]) == 0) return fail(PA_POOL_ERR_INVALID_ARG, "unknown request");
    if (offsets[i + 1] < offsets[i] || offsets[0] != 0 || (offsets[i + 1] > 0 && drafts == nullptr))
      return fail(PA_POOL_ERR_INVALID_ARG, "offsets must start at 0 and not decrease");
  }
  for (int64_t i = 0; i < num_requests; ++i)
    s->drafts[req_ids[i]].assign(drafts + offsets[i], drafts + offsets[i + 1]);
  return PA_POOL_OK;
}

int64_t pa_sched_schedule(pa_scheduler* s) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  std::vector<Item> order;  // scheduling order
  int64_t budget = s->cfg.max_num_batched_tokens;
  bool preempted = false;

  // running requests, oldest first
  size_t i = 0;
  while (i < s->running.size() && budget > 0) {
    const int64_t id = s->running[i];
    const int64_t computed = pa_pool_request_computed(s->pool, id);
    const int64_t lacking = pa_pool_request_tokens(s->pool, id) - computed;
    // draft tokens follow the known ones, as far as the budget goes
    auto dr = s->drafts.find(id);
    const int64_t k = (lacking >= 1 && dr != s->drafts.end()) ? (int64_t)dr->second.size() : 0;
    const int64_t n = std::min(lacking + k, budget);
    const int64_t known = std::min(n, lacking);
    if (n <= 0) {
      ++i;
      continue;
    }
    bool self_preempted = false;
    for (;;) {
      const int st = pa_pool_allocate_slots_lookahead(s->pool, id, known, n - known, nullptr);
      if (st == PA_POOL_OK) break;
      if (st != PA_POOL_NO_SPACE) return fail(st, pa_pool_last_error());
      const size_t v = s->victim_index();
      const int64_t victim = s->running[v];
      s->running.erase(s->running.begin() + v);
      auto it = std::find_if(order.begin(), order.end(), [&](const Item& x) { return x.id == victim; });
      if (it != order.end()) {  // scheduled earlier in this step: take it out again
        budget += it->count;
        order.erase(it);
      }
      bool swapped = false;
      if (s->cfg.preempt_mode == PA_SCHED_SWAP) {
        const int sst = pa_pool_swap_out(s->pool, victim);
        if (sst < 0) return fail(sst, pa_pool_last_error());
        swapped = sst == PA_POOL_OK && pa_pool_request_swapped(s->pool, victim) == 1;
      }
      if (swapped) ++s->swaps;
      else pa_pool_free_request(s->pool, victim, 1);  // recompute later
      s->enqueue_waiting(victim, true);
      ++s->preemptions;
      preempted = true;
      if (victim == id) {
        self_preempted = true;
        break;
      }
      if (v < i) --i;
    }
    if (self_preempted) continue;  // running[i] is now the next request
    order.push_back(Item{id, (int32_t)computed, (int32_t)n, (int32_t)(n - known)});
    budget -= n;
    ++i;
  }

  // waiting requests, in queue order, unless this step preempted
  while (!preempted && !s->waiting.empty() && budget > 0 &&
         (int64_t)s->running.size() < s->cfg.max_num_seqs) {
    const int64_t id = s->waiting.front();
    if (pa_pool_request_swapped(s->pool, id) == 1) {
      // resume at the computed count: swap in, then the blocks of the new tokens
      const int64_t computed = pa_pool_request_computed(s->pool, id);
      const int64_t lacking = pa_pool_request_tokens(s->pool, id) - computed;
      if (!s->cfg.chunked_prefill && lacking > budget) break;
      const int64_t n = std::min(lacking, budget);
      const int64_t held = (computed + 15) / 16;
      const int64_t need = std::max<int64_t>((computed + n + 15) / 16, held);
      if (need > pa_pool_num_free_blocks(s->pool)) break;
      int st = pa_pool_swap_in(s->pool, id);
      if (st == PA_POOL_OK) st = pa_pool_allocate_slots(s->pool, id, n, nullptr);
      if (st != PA_POOL_OK) return fail(st < 0 ? st : PA_POOL_ERR_INVALID_ARG, "swap-in admission failed");
      s->waiting.pop_front();
      s->running.push_back(id);
      order.push_back(Item{id, (int32_t)computed, (int32_t)n, 0});
      budget -= n;
      continue;
    }
    const int64_t hit = pa_pool_prefix_hit_tokens(s->pool, id);
    const int64_t lacking = pa_pool_request_tokens(s->pool, id) - hit;
    if (!s->cfg.chunked_prefill && lacking > budget) break;
    const int64_t n = std::min(lacking, budget);
    const int st = pa_pool_allocate_slots(s->pool, id, n, nullptr);
    if (st == PA_POOL_NO_SPACE) break;
    if (st != PA_POOL_OK) return fail(st, pa_pool_last_error());
    s->waiting.pop_front();
    s->running.push_back(id);
    order.push_back(Item{id, (int32_t)hit, (int32_t)n, 0});
    budget -= n;
  }

  s->plan.clear();
  for (const Item& x : order)
    if (x.count > 1) s->plan.push_back(x);
  // the multi-token requests longest first (ties keep scheduling order), so that
  // short chunks (a request's drafts) end the group and can go to another call
  std::stable_sort(s->plan.begin(), s->plan.end(), [](const Item& a, const Item& b) { return a.count > b.count; });
  for (const Item& x : order)
    if (x.count == 1) s->plan.push_back(x);
  return (int64_t)s->plan.size();
}

int pa_sched_plan(const pa_scheduler* s, int64_t* req_ids, int32_t* starts, int32_t* counts) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  for (size_t i = 0; i < s->plan.size(); ++i) {
    if (req_ids) req_ids[i] = s->plan[i].id;
    if (starts) starts[i] = s->plan[i].start;
    if (counts) counts[i] = s->plan[i].count;
  }
  return PA_POOL_OK;
}

int pa_sched_plan_drafts(const pa_scheduler* s, int32_t* drafts) {
  if (s == nullptr || drafts == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  for (size_t i = 0; i < s->plan.size(); ++i) drafts[i] = s->plan[i].drafts;
  return PA_POOL_OK;
}

int64_t pa_sched_plan_tokens(const pa_scheduler* s) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  int64_t n = 0;
  for (const Item& x : s->plan) n += x.count;
  return n;
}

int64_t pa_sched_plan_prefills(const pa_scheduler* s) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  int64_t n = 0;
  for (const Item& x : s->plan) n += x.count > 1;
  return n;
}

int32_t pa_sched_plan_max_blocks(const pa_scheduler* s) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  int64_t m = 0;
  for (const Item& x : s->plan) m = std::max(m, pa_pool_block_table(s->pool, x.id, nullptr, 0));
  return (int32_t)m;
}

int pa_sched_batch(const pa_scheduler* s, int32_t* query_start_loc, int32_t* seq_lens,
                   int32_t* block_tables, int32_t max_blocks, int32_t pad_block,
                   int32_t* slot_mapping, int32_t* positions) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  if (block_tables != nullptr && max_blocks < pa_sched_plan_max_blocks(s))
    return fail(PA_POOL_ERR_INVALID_ARG, "max_blocks is below the widest block table of the step");
  int32_t q = 0;
  int64_t tok = 0, p = 0;
  if (query_start_loc) query_start_loc[0] = 0;
  for (size_t i = 0; i < s->plan.size(); ++i) {
    const Item& x = s->plan[i];
    if (x.count > 1 && query_start_loc) query_start_loc[++p] = (q += x.count);
    if (seq_lens) seq_lens[i] = x.start + x.count;
    if (block_tables) {
      int32_t* row = block_tables + (int64_t)i * max_blocks;
      const int64_t n = pa_pool_block_table(s->pool, x.id, row, max_blocks);
      for (int64_t j = n; j < max_blocks; ++j) row[j] = pad_block;
    }
    if (slot_mapping) {
      const int st = pa_pool_slot_mapping(s->pool, x.id, x.start, x.count, slot_mapping + tok);
      if (st != PA_POOL_OK) return fail(st, pa_pool_last_error());
    }
    if (positions)
      for (int32_t j = 0; j < x.count; ++j) positions[tok + j] = x.start + j;
    tok += x.count;
  }
  return PA_POOL_OK;
}

int64_t pa_sched_update(pa_scheduler* s, const int32_t* sampled) {
  return pa_sched_update_spec(s, sampled, nullptr);
}

int64_t pa_sched_update_spec(pa_scheduler* s, const int32_t* sampled, const int32_t* num_accepted) {
  if (s == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
  for (size_t i = 0; num_accepted != nullptr && i < s->plan.size(); ++i)
    if (num_accepted[i] < 0 || num_accepted[i] > s->plan[i].drafts)
      return fail(PA_POOL_ERR_INVALID_ARG, "num_accepted[" + std::to_string(i) + "] is outside [0, drafts]");
  int64_t done = 0;
  for (size_t i = 0; i < s->plan.size(); ++i) {
    const Item& x = s->plan[i];
    const int64_t c = (int64_t)x.start + x.count - x.drafts;  // the known tokens computed
    int st = pa_pool_commit(s->pool, x.id, c);
    if (st != PA_POOL_OK) return fail(st, pa_pool_last_error());
    if (c < pa_pool_request_tokens(s->pool, x.id)) continue;  // still catching up
    // generated this step: the accepted drafts, then the token sampled after them
    const int32_t a = num_accepted != nullptr ? num_accepted[i] : 0;
    SchedRequest& r = s->reqs.at(x.id);
    for (int32_t j = 0; j <= a; ++j) {
      if (++r.produced >= r.max_new) {
        pa_pool_free_request(s->pool, x.id, 0);
        s->running.erase(std::find(s->running.begin(), s->running.end(), x.id));
        s->reqs.erase(x.id);
        s->finished.push_back(x.id);
        ++done;
        break;
      }
      if (j < a) {  // an accepted draft: its K/V is in the pool already
        st = pa_pool_append_tokens(s->pool, x.id, &s->drafts.at(x.id)[j], 1);
        if (st == PA_POOL_OK) st = pa_pool_commit(s->pool, x.id, c + j + 1);
      } else {
        if (sampled == nullptr) return fail(PA_POOL_ERR_INVALID_ARG, "sampled tokens needed");
        st = pa_pool_append_tokens(s->pool, x.id, &sampled[i], 1);
      }
      if (st != PA_POOL_OK) return fail(st, pa_pool_last_error());
    }
  }
  s->plan.clear();
  s->drafts.clear();
  return done;
}

int64_t pa_sched_num_waiting(const pa_scheduler* s) {
  return s ? (int64_t)s->waiting.size() : fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
}
int64_t pa_sched_num_running(const pa_scheduler* s) {
  return s ? (int64_t)s->running.size() : fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
}
int64_t pa_sched_num_preemptions(const pa_scheduler* s) {
  return s ? s->preemptions : fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
}
int64_t pa_sched_num_swaps(const pa_scheduler* s) {
  return s ? s->swaps : fail(PA_POOL_ERR_INVALID_ARG, "null scheduler");
}
int64_t pa_sched_take_finished(pa_scheduler* s, int64_t* ids, int64_t max) {
  if (s == nullptr || (max > 0 && ids == nullptr)) return fail(PA_POOL_ERR_INVALID_ARG, "null pointer");
  int64_t n = 0;
  while (n < max && !s->finished.empty()) {
    ids[n++] = s->finished.front();
    s->finished.pop_front();
  }
  return n;
}
const char* pa_sched_last_error(void) { return g_error.c_str(); }

}  // extern "C"
