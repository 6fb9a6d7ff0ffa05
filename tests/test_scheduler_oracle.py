"""Pins of the scheduler model (oracle/scheduler.py) against what the pages state.

Each pin checks one stated behaviour of continuous batching (arcyou teardown of
vLLM paged attention, "Continuous batching: rebuild the batch every step" and
"What happens when the blocks run out") on a small hand-built case, plus an
end-to-end run in which K/V are simulated as token ids: every request always
reads back its own tokens, every request ends with exactly its number of
generated tokens, and the budget is never exceeded. Planted mistakes in the
model must each be caught by at least one pin.
"""
import random

import pytest

from oracle import block_pool as bp
from oracle import scheduler as sm

B = bp.BLOCK


def make(num_blocks, budget, max_seqs=64, policy=sm.FCFS, chunked=True, prefix=True, num_host=0):
    return sm.SchedulerModel(bp.BlockPoolModel(num_blocks, prefix, num_host), budget, max_seqs, policy,
                             chunked, sm.SWAP if num_host else sm.RECOMPUTE)


def apply_ops(ops, dev, hst):
    """Run the pool's block operations in order on simulated device and host contents."""
    for kind, src, dst in ops:
        a, b = {bp.OP_COPY: (dev, dev), bp.OP_SWAP_OUT: (dev, hst), bp.OP_SWAP_IN: (hst, dev)}[kind]
        for o in range(B):
            if src * B + o in a:
                b[dst * B + o] = a[src * B + o]
            else:
                b.pop(dst * B + o, None)


def step(s, dev=None, rng=None, produced=None, hst=None):
    plan = s.schedule()
    ops = s.pool.take_ops()
    if dev is not None:
        apply_ops(ops, dev, {} if hst is None else hst)
    if produced is not None:
        for rid, start, n in plan:
            if start + n == len(s.pool.reqs[rid].tokens):
                produced[rid] = produced.get(rid, 0) + 1
    if dev is not None:
        _, _, _, slots, pos = s.batch()
        k = 0
        for rid, start, n in plan:
            toks = s.pool.reqs[rid].tokens
            for j in range(n):
                dev[slots[k]] = toks[pos[k]]
                k += 1
    sampled = [(rng.randint(0, 99) if rng else 7) for _ in plan]
    s.update(sampled)
    return plan


def readback_ok(s, dev, hst=None):
    for rid, r in s.pool.reqs.items():
        where, blocks = (hst, r.host_blocks) if r.swapped else (dev, r.blocks)
        got = [where.get(blocks[p // B] * B + p % B) for p in range(r.computed)]
        if got != r.tokens[:r.computed]:
            return False
    return True


# ----------------------------------------------------------------------------- pins
def pin_chunked_prefill_splits_a_long_prompt():
    s = make(64, 32)
    s.add_request(1, list(range(100)), 3)
    assert [step(s)[0][2] for _ in range(4)] == [32, 32, 32, 4]
    assert step(s) == [(1, 100, 1)]  # then one token per step


def pin_steps_mix_prompts_and_generation():
    s = make(64, 64)
    s.add_request(1, list(range(20)), 5)
    step(s)
    s.add_request(2, list(range(200, 240)), 5)
    plan = step(s)
    assert sorted(n for _, _, n in plan) == [1, 40]
    assert plan[0][0] == 2  # multi-token requests lead the batch


def pin_running_served_before_waiting():
    s = make(64, 40)
    s.add_request(1, list(range(70)), 2)
    step(s)                                  # 40 of 70
    s.add_request(2, list(range(100, 110)), 2)
    plan = step(s)
    assert plan[0] == (1, 40, 30) and (2, 0, 10) in plan


def pin_budget_is_never_exceeded():
    rng = random.Random(3)
    s = make(40, 24)
    for i in range(12):
        s.add_request(i, [rng.randint(0, 9) for _ in range(rng.randint(1, 60))], rng.randint(1, 6))
    for _ in range(200):
        plan = step(s, rng=rng)
        assert sum(n for _, _, n in plan) <= 24


def pin_preemption_takes_the_newest_and_requeues_it_first():
    s = make(6, 64)
    s.add_request(1, list(range(40)), 30)    # 3 blocks
    s.add_request(2, list(range(100, 140)), 30)  # 3 blocks: the pool is full
    step(s)
    s.add_request(3, [5, 5], 1)
    for _ in range(30):                      # request 1 needs a 4th block at position 48
        step(s)
        if s.preemptions:
            break
    assert s.preemptions == 1
    assert s.running == [1] and s.waiting == [2, 3] and s.pool.reqs[2].computed == 0
    assert s.pool.prefix_hit_tokens(2) >= 32  # its prefix survived in the pool


def pin_priority_preempts_lowest_priority_latest_arrival():
    s = make(6, 64, policy=sm.PRIORITY)
    s.add_request(1, list(range(40)), 30, priority=5)
    s.add_request(2, list(range(100, 140)), 30, priority=0)
    step(s)
    for _ in range(30):
        step(s)
        if s.preemptions:
            break
    assert s.preemptions == 1 and s.running == [2] and s.waiting == [1]


def pin_swap_mode_resumes_where_it_stopped():
    """Same trace as the FCFS preemption pin, with a swap space: the victim keeps its computed
    tokens in host memory and resumes from them, so it is never recomputed."""
    s = make(6, 64, num_host=4)
    s.add_request(1, list(range(40)), 30)
    s.add_request(2, list(range(100, 140)), 30)
    step(s)
    for _ in range(30):
        step(s)
        if s.preemptions:
            break
    r2 = s.pool.reqs[2]
    assert s.swaps == 1 and r2.swapped and r2.computed > 40 and s.waiting == [2]
    computed = r2.computed
    for _ in range(200):
        plan = step(s)
        mine = [x for x in plan if x[0] == 2]
        if mine:
            assert mine[0][1] == computed  # resumes at its computed count
            break
    else:
        raise AssertionError("swapped request never resumed")


def pin_swap_mode_without_room_recomputes():
    s = make(6, 64, num_host=2)  # request 2 needs 3 host blocks
    s.add_request(1, list(range(40)), 30)
    s.add_request(2, list(range(100, 140)), 30)
    step(s)
    for _ in range(30):
        step(s)
        if s.preemptions:
            break
    assert s.preemptions == 1 and s.swaps == 0 and s.pool.reqs[2].computed == 0


def pin_finished_requests_release_their_blocks():
    s = make(8, 64)
    s.add_request(1, list(range(30)), 1)
    step(s)
    assert s.finished == [1] and len(s.pool.free) == 8 and s.running == []


def pin_no_admission_beyond_max_seqs():
    s = make(64, 64, max_seqs=2)
    for i in range(4):
        s.add_request(i, [i] * 5, 3)
    plan = step(s)
    assert [rid for rid, _, _ in plan] == [0, 1] and s.waiting == [2, 3]


def pin_without_chunking_a_prompt_waits_for_room():
    s = make(64, 32, chunked=False)
    s.add_request(1, list(range(20)), 4)
    s.add_request(2, list(range(50)), 4)
    plan = step(s)
    assert [rid for rid, _, _ in plan] == [1] and s.waiting == [2]


def pin_trace_completes_and_reads_back():
    for seed in range(16):
        rng = random.Random(seed)
        s = make(rng.choice([8, 12, 40]), rng.choice([16, 48]), max_seqs=rng.choice([2, 8]),
                 policy=rng.choice([sm.FCFS, sm.PRIORITY]), num_host=rng.choice([0, 0, 3, 10]))
        dev, hst, produced, max_new = {}, {}, {}, {}
        shared = [rng.randint(0, 9) for _ in range(32)]
        for i in range(10):
            prompt = (shared if rng.random() < 0.5 else []) + [rng.randint(0, 9) for _ in range(rng.randint(1, 40))]
            max_new[i] = rng.randint(1, 8)
            s.add_request(i, prompt, max_new[i], priority=rng.randint(0, 2))
        for _ in range(2000):
            step(s, dev, rng, produced, hst)
            assert readback_ok(s, dev, hst)
            if not s.running and not s.waiting:
                break
        assert sorted(s.finished) == list(range(10))
        assert produced == max_new


# ---- speculative tokens: a request is (tokens computed, tokens known plus drafts)

def spec_step(s, dev, rng, produced, max_new):
    """One step with random drafts (0-3 tokens, ids 100-109, never a sampled id) for every
    running request and a random number of them accepted; the simulated device gets every
    scheduled position's token id, drafts included."""
    for rid in list(s.running):
        s.set_spec_tokens(rid, [rng.randint(100, 109) for _ in range(rng.randint(0, 3))])
    plan = s.schedule()
    apply_ops(s.pool.take_ops(), dev, {})
    _, _, _, slots, pos = s.batch()
    k = 0
    accepted = []
    for (rid, start, n), d in zip(plan, s.plan_drafts):
        toks = s.pool.reqs[rid].tokens + s.drafts.get(rid, [])[:d]
        for j in range(n):
            dev[slots[k]] = toks[pos[k]]
            k += 1
        a = rng.randint(0, d)
        accepted.append(a)
        if start + n - d == len(s.pool.reqs[rid].tokens):
            produced[rid] = min(produced.get(rid, 0) + a + 1, max_new[rid])
    assert sum(n for _, _, n in plan) <= s.budget
    s.update([rng.randint(0, 99) for _ in plan], accepted)
    return plan


def pin_drafts_follow_the_known_tokens():
    s = make(64, 64)
    s.add_request(1, list(range(20)), 9)
    step(s)                                       # the prompt; 7 is sampled
    s.set_spec_tokens(1, [101, 102, 103])
    assert s.schedule() == [(1, 20, 4)] and s.plan_drafts == [3]
    _, seq, _, slots, pos = s.batch()
    assert seq == [24] and pos == [20, 21, 22, 23]
    s.update([9], [2])                            # two drafts accepted, then 9 sampled
    r = s.pool.reqs[1]
    assert r.tokens == list(range(20)) + [7, 101, 102, 9] and r.computed == 23
    assert s.schedule() == [(1, 23, 1)] and s.plan_drafts == [0]  # drafts last one step


def pin_drafts_fit_the_budget():
    s = make(64, 3)
    s.add_request(1, [5], 9)
    step(s)
    s.set_spec_tokens(1, [101, 102, 103, 104])
    assert s.schedule() == [(1, 1, 3)] and s.plan_drafts == [2]
    s.update([9], [0])                            # none accepted: only the sampled token
    assert s.pool.reqs[1].tokens == [5, 7, 9] and s.pool.reqs[1].computed == 2


def pin_a_prompt_catching_up_gets_no_drafts():
    s = make(64, 32)
    s.add_request(1, list(range(100)), 3)
    s.set_spec_tokens(1, [101])
    assert s.schedule() == [(1, 0, 32)] and s.plan_drafts == [0]


def pin_accepted_drafts_count_as_generated():
    s = make(64, 64)
    s.add_request(1, list(range(20)), 3)
    step(s)                                       # first generated token
    s.set_spec_tokens(1, [101, 102, 103])
    s.schedule()
    assert s.update([9], [3]) == 1                # 101, 102 make 3: finished, 102 not appended
    assert s.finished == [1] and 1 not in s.pool.reqs


def pin_spec_trace_reads_back():
    """Random drafts and acceptance: every computed position holds its token (a rejected
    draft is never counted as computed), and every request makes exactly its tokens."""
    for seed in range(16):
        rng = random.Random(100 + seed)
        s = make(rng.choice([10, 16, 40]), rng.choice([8, 24, 48]), max_seqs=rng.choice([2, 8]),
                 policy=rng.choice([sm.FCFS, sm.PRIORITY]))
        dev, produced, max_new = {}, {}, {}
        for i in range(10):
            max_new[i] = rng.randint(1, 12)
            s.add_request(i, [rng.randint(0, 99) for _ in range(rng.randint(1, 40))], max_new[i],
                          priority=rng.randint(0, 2))
        for _ in range(2000):
            spec_step(s, dev, rng, produced, max_new)
            assert readback_ok(s, dev)
            if not s.running and not s.waiting:
                break
        assert sorted(s.finished) == list(range(10))
        assert produced == max_new


ALL_PINS = [pin_chunked_prefill_splits_a_long_prompt, pin_steps_mix_prompts_and_generation,
            pin_running_served_before_waiting, pin_budget_is_never_exceeded,
            pin_preemption_takes_the_newest_and_requeues_it_first,
            pin_priority_preempts_lowest_priority_latest_arrival,
            pin_finished_requests_release_their_blocks, pin_no_admission_beyond_max_seqs,
            pin_swap_mode_resumes_where_it_stopped, pin_swap_mode_without_room_recomputes,
            pin_without_chunking_a_prompt_waits_for_room, pin_trace_completes_and_reads_back,
            pin_drafts_follow_the_known_tokens, pin_drafts_fit_the_budget,
            pin_a_prompt_catching_up_gets_no_drafts, pin_accepted_drafts_count_as_generated,
            pin_spec_trace_reads_back]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


MISTAKES = {
    "preempt the oldest": ("victim", lambda self: self.running[0]),
    "preempted request to the tail": ("enqueue", lambda self, rid, pre: self.waiting.append(rid)),
    "priority ignored when preempting": ("rank", lambda self, rid: (0, self.info[rid]["arrival"])),
}


def _plan_order_decodes_first(self):
    plan = _orig_schedule(self)
    self.plan = [x for x in plan if x[2] == 1] + [x for x in plan if x[2] > 1]
    return list(self.plan)


def _no_chunking(self):
    self.chunked = False
    saved, self.budget = self.budget, 10 ** 9
    try:
        return _orig_schedule(self)
    finally:
        self.budget = saved


def _keep_finished_blocks(self, sampled, accepted=None):
    free = self.pool.free_request
    self.pool.free_request = lambda rid, keep=False: None if not keep else free(rid, keep)
    try:
        return _orig_update(self, sampled, accepted)
    finally:
        self.pool.free_request = free


def _rejected_drafts_committed(self, sampled, accepted=None):
    # every scheduled position counted as computed once the tokens reach it: the
    # sampled token's position then claims the first rejected draft's K/V
    plan = list(self.plan)
    done = _orig_update(self, sampled, accepted)
    for rid, start, n in plan:
        r = self.pool.reqs.get(rid)
        if r is not None:
            self.pool.commit(rid, max(r.computed, min(start + n, len(r.tokens), 16 * len(r.blocks))))
    return done


def _drafts_ignore_the_budget(self):
    saved = self.budget
    extra = sum(len(d) for d in self.drafts.values())
    self.budget = saved + extra  # the drafts come on top of the budget
    try:
        return _orig_schedule(self)
    finally:
        self.budget = saved


def _swap_ignored(self):
    self.preempt_mode = sm.RECOMPUTE
    return _orig_schedule(self)


_orig_schedule = sm.SchedulerModel.schedule
_orig_update = sm.SchedulerModel.update
MISTAKES.update({
    "decodes lead the batch": ("schedule", _plan_order_decodes_first),
    "whole prompts ignore the budget": ("schedule", _no_chunking),
    "finished requests keep their blocks": ("update", _keep_finished_blocks),
    "swap mode recomputes instead": ("schedule", _swap_ignored),
    "rejected drafts counted as computed": ("update", _rejected_drafts_committed),
    "drafts on top of the budget": ("schedule", _drafts_ignore_the_budget),
})


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, wrong = MISTAKES[name]
    monkeypatch.setattr(sm.SchedulerModel, attr, wrong)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, f"no pin noticed the planted mistake {name!r}"
