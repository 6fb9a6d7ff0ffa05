"""Plain Python model of the continuous-batching step scheduler.

TEST INFRASTRUCTURE. Only the tests may import this module; the library and its
binding never do. It drives the block-pool model of oracle/block_pool.py.

Rules and where they come from (arcyou teardown of vLLM paged attention,
sections "Continuous batching: rebuild the batch every step" and "What happens
when the blocks run out"):
  * There are no prefill and decode phases: a request is (tokens computed,
    tokens known), and each step hands out a token budget.
  * Running requests are served first, then waiting ones are admitted until the
    budget runs out; a long prompt is split over steps (chunked prefill).
  * When the pool cannot grow a request, the newest running request is preempted
    (FCFS), or the lowest-priority, latest-arrival one (priority scheduling); its
    blocks are freed, its computed count reset to 0, and it goes back to the head
    of the waiting queue to be recomputed.
  * A finished request frees its blocks at once.
  * The preempted request may instead keep its K/V by swapping it to CPU memory
    (aitrending, "The 1960s Operating System Trick That Makes vLLM 4x Faster",
    Technical Details: swap or recompute).
  * A request is a pair (tokens computed, tokens known plus speculative tokens):
    a running request may carry draft tokens for the next step, which the step
    computes after its known tokens, budget permitting.

Readings where the pages are silent (the same as the library's): no admission
in a step that preempted; without chunked prefill, admission stops at the first
waiting request whose remaining tokens exceed the budget left; under priority
scheduling the waiting queue is kept in (priority, arrival) order and a victim
already scheduled in the step is taken out of it; a request finishes on its
max_new_tokens-th generated token, which is not appended; the batch lists the
requests given more than one token first, the longest first, then the one-token
ones (short chunks, such as a request's drafts, then sit together at the end of
the multi-token group); in swap mode
the victim is swapped out when the swap space has room (else recomputed), and a
swapped request is admitted only when the free queue covers its swap-in and the
blocks of the tokens it is given, resuming at its computed count. Drafts: they
are set for one step and dropped at its update; only a running request whose
known tokens all fit the step gets them (as many as the budget leaves), and its
blocks then cover them too; the update takes, per request, how many of the
scheduled drafts were accepted (a prefix of them) and the token sampled after
the last accepted one; the accepted drafts join the request's tokens as
computed (their K/V was written by the step), then the sampled token is
appended; each of these counts as one generated token, and the request
finishes at its max_new_tokens-th as before (that token is not appended, and
the rest of the step's tokens for it are dropped). Rejected drafts leave K/V in
slots past the computed count, which later steps overwrite.
"""
from __future__ import annotations

from .block_pool import BlockPoolModel

FCFS, PRIORITY = 0, 1
RECOMPUTE, SWAP = 0, 1


class SchedulerModel:
    def __init__(self, pool: BlockPoolModel, max_num_batched_tokens: int, max_num_seqs: int,
                 policy: int = FCFS, chunked_prefill: bool = True, preempt_mode: int = RECOMPUTE):
        self.pool = pool
        self.budget = max_num_batched_tokens
        self.max_seqs = max_num_seqs
        self.policy = policy
        self.chunked = chunked_prefill
        self.info = {}       # id -> dict(max_new, priority, arrival, produced)
        self.waiting = []    # head first
        self.running = []    # start order
        self.plan = []       # (id, start, count), batch order
        self.drafts = {}     # id -> draft tokens for the next step
        self.plan_drafts = []  # drafts scheduled per plan item (the last ones of its count)
        self.finished = []
        self.preemptions = 0
        self.swaps = 0
        self.preempt_mode = preempt_mode
        self.arrivals = 0

    # ---------------------------------------------------------------- rules
    def rank(self, rid):
        i = self.info[rid]
        return (i["priority"], i["arrival"])

    def enqueue(self, rid, preempted):
        if self.policy == PRIORITY:
            k = 0
            while k < len(self.waiting) and self.rank(self.waiting[k]) <= self.rank(rid):
                k += 1
            self.waiting.insert(k, rid)
        elif preempted:
            self.waiting.insert(0, rid)
        else:
            self.waiting.append(rid)

    def victim(self):
        if self.policy == PRIORITY:
            return max(self.running, key=self.rank)
        return self.running[-1]

    # ---------------------------------------------------------------- calls
    def add_request(self, rid, prompt, max_new_tokens, priority=0, salt=0):
        self.pool.add_request(rid, prompt, salt)
        self.info[rid] = dict(max_new=max_new_tokens, priority=priority, arrival=self.arrivals, produced=0)
        self.arrivals += 1
        self.enqueue(rid, False)

    def set_spec_tokens(self, rid, drafts):
        if rid not in self.info:
            raise ValueError("unknown request")
        self.drafts[rid] = list(drafts)

    def schedule(self):
        order = []
        look = {}  # id -> drafts scheduled
        budget = self.budget
        preempted = False
        i = 0
        while i < len(self.running) and budget > 0:
            rid = self.running[i]
            r = self.pool.reqs[rid]
            start = r.computed
            real = len(r.tokens) - start
            k = len(self.drafts.get(rid, ())) if real >= 1 else 0
            n = min(real + k, budget)
            if n <= 0:
                i += 1
                continue
            gone = False
            while self.pool.allocate_slots(rid, min(n, real), n - min(n, real)) is None:
                v = self.victim()
                vi = self.running.index(v)
                self.running.remove(v)
                for item in order:
                    if item[0] == v:
                        budget += item[2]
                        order.remove(item)
                        break
                if self.preempt_mode == SWAP and self.pool.swap_out(v) and self.pool.reqs[v].swapped:
                    self.swaps += 1
                else:
                    self.pool.free_request(v, keep=True)
                self.enqueue(v, True)
                self.preemptions += 1
                preempted = True
                if v == rid:
                    gone = True
                    break
                if vi < i:
                    i -= 1
            if gone:
                continue
            order.append((rid, start, n))
            look[rid] = n - min(n, real)
            budget -= n
            i += 1
        while (not preempted and self.waiting and budget > 0
               and len(self.running) < self.max_seqs):
            rid = self.waiting[0]
            r = self.pool.reqs[rid]
            if r.swapped:
                lacking = len(r.tokens) - r.computed
                if not self.chunked and lacking > budget:
                    break
                n = min(lacking, budget)
                held = -(-r.computed // 16)
                if max(-(-(r.computed + n) // 16), held) > len(self.pool.free):
                    break
                start = r.computed
                assert self.pool.swap_in(rid) and self.pool.allocate_slots(rid, n) is not None
                self.waiting.pop(0)
                self.running.append(rid)
                order.append((rid, start, n))
                budget -= n
                continue
            hit = self.pool.prefix_hit_tokens(rid)
            lacking = len(self.pool.reqs[rid].tokens) - hit
            if not self.chunked and lacking > budget:
                break
            n = min(lacking, budget)
            if self.pool.allocate_slots(rid, n) is None:
                break
            self.waiting.pop(0)
            self.running.append(rid)
            order.append((rid, hit, n))
            budget -= n
        # multi-token requests first, the longest first (ties in scheduling order), then
        # the one-token ones in scheduling order
        self.plan = sorted([x for x in order if x[2] > 1], key=lambda x: -x[2]) + [x for x in order if x[2] == 1]
        self.plan_drafts = [look.get(x[0], 0) for x in self.plan]
        return list(self.plan)

    def batch(self, pad_block=0):
        """query_start_loc, seq_lens, block tables, slot mapping, positions of the plan."""
        qsl = [0]
        seq, tables, slots, pos = [], [], [], []
        width = max([len(self.pool.reqs[rid].blocks) for rid, _, _ in self.plan] + [1])
        for rid, start, n in self.plan:
            if n > 1:
                qsl.append(qsl[-1] + n)
            seq.append(start + n)
            t = self.pool.block_table(rid)
            tables.append(t + [pad_block] * (width - len(t)))
            slots += self.pool.slot_mapping(rid, start, n)
            pos += list(range(start, start + n))
        return qsl, seq, tables, slots, pos

    def update(self, sampled, accepted=None):
        """accepted[i]: how many of plan item i's scheduled drafts were accepted (None: none)."""
        done = 0
        for i, (rid, start, n) in enumerate(self.plan):
            d = self.plan_drafts[i]
            a = 0 if accepted is None else accepted[i]
            if not 0 <= a <= d:
                raise ValueError("accepted drafts out of range")
            r = self.pool.reqs[rid]
            c = start + n - d  # the known tokens computed
            self.pool.commit(rid, c)
            if c < len(r.tokens):
                continue
            info = self.info[rid]
            outs = self.drafts[rid][:a] + [sampled[i]] if a else [sampled[i]]
            for j, t in enumerate(outs):
                info["produced"] += 1
                if info["produced"] >= info["max_new"]:
                    self.pool.free_request(rid)
                    self.running.remove(rid)
                    del self.info[rid]
                    self.finished.append(rid)
                    done += 1
                    break
                self.pool.append_tokens(rid, [t])
                if j < a:  # an accepted draft: its K/V is in the pool already
                    self.pool.commit(rid, c + j + 1)
        self.plan = []
        self.plan_drafts = []
        self.drafts = {}
        return done
