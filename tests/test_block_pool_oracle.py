"""Pins of the block-pool model (oracle/block_pool.py) against what the pages state.

Each pin checks one stated behaviour of the paged KV memory (arcyou teardown of
vLLM paged attention, "PagedAttention: the KV cache is paged, like virtual
memory" and "What happens when the blocks run out"; aitrending, "The 1960s
Operating System Trick That Makes vLLM 4x Faster", Technical Details) on small
hand-built cases, plus one end-to-end invariant: with K/V simulated as the token
ids themselves, every request reads back exactly its own tokens through its
block table after any sequence of allocations, forks, copies and frees. Planted
mistakes in the model must each be caught by at least one pin.
"""
import random

import pytest

from oracle import block_pool as bp

B = bp.BLOCK


def tokens(n, base=0):
    return [base + i for i in range(n)]


def apply_ops(ops, device, host=None):
    """Run block operations in order on the simulated device (and host) contents."""
    host = {} if host is None else host
    for kind, src, dst in ops:
        a, b = {bp.OP_COPY: (device, device), bp.OP_SWAP_OUT: (device, host),
                bp.OP_SWAP_IN: (host, device)}[kind]
        for o in range(B):
            if src * B + o in a:
                b[dst * B + o] = a[src * B + o]
            else:
                b.pop(dst * B + o, None)


def run_chunk(pool, rid, n, device, host=None):
    """Schedule n tokens of rid: allocate, run the queued block operations, write, commit."""
    r = pool.reqs[rid]
    hit = pool.allocate_slots(rid, n)
    if hit is None:
        return None
    apply_ops(pool.take_ops(), device, host)
    start = r.computed
    for p, slot in zip(range(start, start + n), pool.slot_mapping(rid, start, n)):
        device[slot] = r.tokens[p]
    pool.commit(rid, start + n)
    return hit


def readback(pool, rid, device, host=None):
    r = pool.reqs[rid]
    where, blocks = (host, r.host_blocks) if r.swapped else (device, r.blocks)
    return [where.get(blocks[p // B] * B + p % B) for p in range(r.computed)]


# ----------------------------------------------------------------------------- pins
def pin_new_request_takes_ceil_blocks():
    for n in range(1, 70):
        pool = bp.BlockPoolModel(8, True)
        pool.add_request(1, tokens(n))
        assert pool.allocate_slots(1, n) == 0
        assert len(pool.block_table(1)) == -(-n // B)
        assert len(pool.free) == 8 - -(-n // B)


def pin_lookahead_blocks_cover_the_drafts():
    """Blocks for positions past the known tokens (speculative drafts): the table covers
    them and their slots are addressable, but they never count as computed."""
    pool = bp.BlockPoolModel(8, True)
    pool.add_request(1, tokens(15))
    assert pool.allocate_slots(1, 15, 2) == 0
    assert len(pool.block_table(1)) == 2 and len(pool.slot_mapping(1, 15, 2)) == 2
    pool.commit(1, 15)
    with pytest.raises(ValueError):
        pool.commit(1, 17)  # the drafts are not tokens of the request
    pool.append_tokens(1, [3])
    pool.commit(1, 16)      # an accepted draft becomes a computed token
    assert pool.reqs[1].computed == 16 and pool.num_cached() == 1
    free = list(pool.free)
    assert pool.allocate_slots(1, 0, 16 * 7 + 1) is None  # 9 blocks in all: 7 more, 6 free
    assert pool.free == free and len(pool.block_table(1)) == 2
    assert pool.allocate_slots(1, 0, 16 * 7) == 0 and pool.free == []


def pin_exhaustion_returns_none_and_changes_nothing():
    pool = bp.BlockPoolModel(4, True)
    pool.add_request(1, tokens(65))
    before = (list(pool.free), list(pool.ref))
    assert pool.allocate_slots(1, 65) is None
    assert (pool.free, pool.ref, pool.block_table(1)) == (before[0], before[1], [])
    pool.add_request(2, tokens(64))
    assert pool.allocate_slots(2, 64) == 0 and pool.free == []


def pin_identical_prompts_share_blocks():
    pool = bp.BlockPoolModel(16, True)
    dev = {}
    prompt = tokens(48, 1000)
    pool.add_request(1, prompt + [1, 2, 3])
    run_chunk(pool, 1, 51, dev)
    free_before = len(pool.free)
    pool.add_request(2, prompt + [7, 8])
    assert pool.prefix_hit_tokens(2) == 48
    assert run_chunk(pool, 2, 2, dev) == 48
    assert pool.block_table(2)[:3] == pool.block_table(1)[:3]
    assert all(pool.ref[b] == 2 for b in pool.block_table(1)[:3])
    assert len(pool.free) == free_before - 1  # only the new tail block
    assert readback(pool, 2, dev) == prompt + [7, 8]


def pin_hash_covers_the_whole_prefix():
    pool = bp.BlockPoolModel(16, True)
    dev = {}
    x, y, z = tokens(B, 0), tokens(B, 100), tokens(B, 200)
    pool.add_request(1, x + y + [5])
    run_chunk(pool, 1, 2 * B + 1, dev)
    pool.add_request(2, z + y + [5])  # same second block content, other prefix
    assert pool.prefix_hit_tokens(2) == 0
    pool.add_request(3, x + z + [5])  # same first block only
    assert pool.prefix_hit_tokens(3) == B
    pool.add_request(4, y + [5])  # y cached only as a second block: its K/V depend on x
    assert pool.prefix_hit_tokens(4) == 0


def pin_extra_key_separates():
    pool = bp.BlockPoolModel(16, True)
    dev = {}
    pool.add_request(1, tokens(40), salt=1)
    run_chunk(pool, 1, 40, dev)
    pool.add_request(2, tokens(40), salt=2)
    assert pool.prefix_hit_tokens(2) == 0
    pool.add_request(3, tokens(40), salt=1)
    assert pool.prefix_hit_tokens(3) == 32


def pin_block_returns_only_at_zero_refs():
    pool = bp.BlockPoolModel(16, True)
    dev = {}
    pool.add_request(1, tokens(33))
    run_chunk(pool, 1, 33, dev)
    pool.add_request(2, tokens(33))
    run_chunk(pool, 2, 1, dev)
    shared = pool.block_table(1)[:2]
    pool.free_request(1)
    assert all(b not in pool.free and pool.ref[b] == 1 for b in shared)
    pool.free_request(2)
    assert all(b in pool.free and pool.ref[b] == 0 for b in shared)


def pin_cached_blocks_evicted_last_prefix_last():
    pool = bp.BlockPoolModel(8, True)
    dev = {}
    pool.add_request(1, tokens(4 * B + 3))
    run_chunk(pool, 1, 4 * B + 3, dev)
    t = pool.block_table(1)  # 4 full cached blocks + 1 partial
    pool.free_request(1)
    # the partial block has nothing to keep: head; cached ones at the tail, last block first
    assert pool.free[0] == t[4]
    assert pool.free[-4:] == [t[3], t[2], t[1], t[0]]
    # use up every uncached block and one cached block: the request's last full block goes
    pool.add_request(2, tokens(4 * B + 1, 500))
    run_chunk(pool, 2, 4 * B + 1, dev)
    assert t[3] in pool.block_table(2) and t[0] not in pool.block_table(2)
    pool.add_request(3, tokens(4 * B + 3))
    assert pool.prefix_hit_tokens(3) == 3 * B


def pin_preempted_request_gets_its_prefix_back():
    pool = bp.BlockPoolModel(16, True)
    dev = {}
    pool.add_request(1, tokens(50))
    run_chunk(pool, 1, 40, dev)
    pool.free_request(1, keep=True)
    assert pool.reqs[1].computed == 0 and pool.block_table(1) == []
    assert pool.prefix_hit_tokens(1) == 32
    assert run_chunk(pool, 1, 18, dev) == 32
    assert readback(pool, 1, dev) == tokens(50)


def pin_last_token_is_always_computed():
    pool = bp.BlockPoolModel(16, True)
    dev = {}
    pool.add_request(1, tokens(2 * B))
    run_chunk(pool, 1, 2 * B, dev)
    pool.add_request(2, tokens(2 * B))
    assert pool.prefix_hit_tokens(2) == B
    assert run_chunk(pool, 2, B, dev) == B


def pin_no_caching_when_disabled():
    pool = bp.BlockPoolModel(16, False)
    dev = {}
    pool.add_request(1, tokens(40))
    run_chunk(pool, 1, 40, dev)
    pool.add_request(2, tokens(40))
    assert pool.prefix_hit_tokens(2) == 0 and pool.num_cached() == 0


def pin_swap_keeps_the_computed_tokens():
    pool = bp.BlockPoolModel(8, True, num_host_blocks=3)
    dev, hst = {}, {}
    pool.add_request(1, tokens(45))
    run_chunk(pool, 1, 37, dev)
    t = pool.block_table(1)
    assert pool.swap_out(1) is True
    ops = pool.take_ops()
    assert ops == [(bp.OP_SWAP_OUT, t[0], 0), (bp.OP_SWAP_OUT, t[1], 1), (bp.OP_SWAP_OUT, t[2], 2)]
    apply_ops(ops, dev, hst)
    assert pool.reqs[1].swapped and pool.reqs[1].computed == 37 and len(pool.free) == 8
    for b in t:                          # someone else overwrites the old blocks
        for o in range(B):
            dev[b * B + o] = -1
    assert pool.swap_in(1) is True and pool.host_free == [0, 1, 2]
    apply_ops(pool.take_ops(), dev, hst)
    assert readback(pool, 1, dev) == tokens(37)
    assert run_chunk(pool, 1, 8, dev) == 0
    assert readback(pool, 1, dev) == tokens(45)
    pool.add_request(2, tokens(70, 500))
    run_chunk(pool, 2, 60, dev)
    assert pool.swap_out(2) is False     # 4 blocks hold computed tokens, 3 host blocks
    assert not pool.reqs[2].swapped and len(pool.reqs[2].blocks) == 4


def pin_reads_back_own_tokens_under_random_use():
    """Fork, diverge, preempt (recompute or swap), finish at random: every request reads
    back its tokens, with copies and swaps run in the order the pool queued them."""
    for seed in range(30):
        rng = random.Random(seed)
        pool = bp.BlockPoolModel(rng.choice([6, 10, 24]), True, num_host_blocks=rng.choice([0, 4, 12]))
        dev, hst = {}, {}
        next_id = 0
        vocab = [tokens(B, 0), tokens(B, 50), tokens(B, 90)]
        for _ in range(120):
            op = rng.random()
            live = sorted(pool.reqs)
            if op < 0.2 or not live:
                prompt = sum((rng.choice(vocab) for _ in range(rng.randint(0, 3))), [])
                prompt += [rng.randint(1000, 1010) for _ in range(rng.randint(1, 20))]
                pool.add_request(next_id, prompt, salt=rng.randint(0, 1))
                next_id += 1
            elif op < 0.55:
                rid = rng.choice(live)
                r = pool.reqs[rid]
                if r.swapped:
                    if pool.swap_in(rid):
                        apply_ops(pool.take_ops(), dev, hst)
                    continue
                left = len(r.tokens) - r.computed - pool.prefix_hit_tokens(rid)
                if left <= 0:
                    pool.append_tokens(rid, [rng.randint(2000, 2100)])
                    left = 1
                run_chunk(pool, rid, rng.randint(1, left), dev, hst)
            elif op < 0.7:
                rid = rng.choice(live)
                if pool.reqs[rid].computed and not pool.reqs[rid].swapped:
                    pool.fork(rid, next_id)
                    pool.append_tokens(next_id, [rng.randint(3000, 3100)])
                    pool.append_tokens(rid, [rng.randint(4000, 4100)])
                    next_id += 1
            elif op < 0.8:
                rid = rng.choice(live)
                if not pool.reqs[rid].swapped and pool.swap_out(rid):
                    apply_ops(pool.take_ops(), dev, hst)
            elif op < 0.9:
                pool.free_request(rng.choice(live), keep=rng.random() < 0.5)
            for rid in pool.reqs:
                assert readback(pool, rid, dev, hst) == pool.reqs[rid].tokens[:pool.reqs[rid].computed]
            held = sum(pool.ref)
            assert held == sum(len(r.blocks) for r in pool.reqs.values())
            assert sorted(pool.free + [b for b in range(len(pool.ref)) if pool.ref[b]]) == \
                list(range(len(pool.ref)))


ALL_PINS = [pin_swap_keeps_the_computed_tokens, pin_new_request_takes_ceil_blocks, pin_exhaustion_returns_none_and_changes_nothing,
            pin_identical_prompts_share_blocks, pin_hash_covers_the_whole_prefix,
            pin_extra_key_separates, pin_block_returns_only_at_zero_refs,
            pin_cached_blocks_evicted_last_prefix_last, pin_preempted_request_gets_its_prefix_back,
            pin_last_token_is_always_computed, pin_no_caching_when_disabled,
            pin_reads_back_own_tokens_under_random_use, pin_lookahead_blocks_cover_the_drafts]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def _partial_allocate(self, rid, n_new, lookahead=0):
    r = self.reqs[rid]
    while len(r.blocks) < bp.ceil_blocks(r.computed + n_new + lookahead) and self.free:
        r.blocks.append(self.take_head())
    return 0


def _swap_out_without_ops(self, rid):
    ok = _orig_swap_out(self, rid)
    self.ops = [o for o in self.ops if o[0] != bp.OP_SWAP_OUT]
    return ok


def _swap_in_reversed(self, rid):
    self.reqs[rid].host_blocks.reverse()
    return _orig_swap_in(self, rid)


_orig_swap_out = bp.BlockPoolModel.swap_out
_orig_swap_in = bp.BlockPoolModel.swap_in

MISTAKES = {
    "hash of the block alone": ("prefix_key", lambda self, r, i: (r.salt, tuple(r.tokens[B * i:B * (i + 1)]))),
    "extra key ignored": ("prefix_key", lambda self, r, i: tuple(r.tokens[:B * (i + 1)])),
    "freed blocks all to the head": ("requeue", lambda self, b: self.free.insert(0, b)),
    "freed blocks all to the tail": ("requeue", lambda self, b: self.free.append(b)),
    "released first block first": ("release_order", lambda self, blocks: list(blocks)),
    "hit may cover the last token": ("max_hit_blocks", lambda self, r: len(r.tokens) // B),
    "no copy on write": ("needs_copy", lambda self, r, start, n: False),
    "partial allocation instead of None": ("allocate_slots", _partial_allocate),
    "swap-out moves nothing": ("swap_out", _swap_out_without_ops),
    "swap-in reverses the blocks": ("swap_in", _swap_in_reversed),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, wrong = MISTAKES[name]
    monkeypatch.setattr(bp.BlockPoolModel, attr, wrong)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure counts
            failed.append(pin.__name__)
    assert failed, f"no pin noticed the planted mistake {name!r}"
