"""Plain Python model of the host KV block pool with prefix caching.

TEST INFRASTRUCTURE. Only the tests may import this module; the library and its
binding never do, and it imports nothing from them.

What the pool does, and where each rule comes from (arcyou teardown of vLLM
paged attention, section "PagedAttention: the KV cache is paged, like virtual
memory", unless noted):
  * KV memory is a fixed set of 16-token blocks; a request holds a list of
    block ids, and room for new tokens is taken as whole blocks off a free
    queue. When the free queue cannot cover the request the call returns None
    and changes nothing (same page, section "What happens when the blocks run
    out", is where the caller reacts by preempting).
  * Each full block is identified by its whole prefix: the hash chains the
    parent block's hash with this block's token ids and extra keys. This model
    uses the exact key (extra key, every token up to the block's end) in place
    of a hash, which is what the chained hash stands for.
  * A request whose prefix matches cached blocks takes a reference on them (no
    copy). A block goes back to the free queue only when its reference count
    reaches zero; cached free blocks sit at the tail, so they are evicted last.
    A request is released tail block first, so its prefix blocks are the last
    of its blocks to be evicted, and a preempted request can find its prefix
    again when it is scheduled anew.
  * Forked requests share blocks until one writes into a shared block; that
    block is copied first (aitrending, "The 1960s Operating System Trick That
    Makes vLLM 4x Faster", Technical Details, copy-on-write).
  * A preempted request may keep its K/V by swapping its blocks to CPU memory
    and swapping them back when it resumes (same page and section).

Readings where the pages are silent (the same as the library's):
  * Blocks needed = ceil(tokens the request will hold / 16) - blocks it holds.
  * The free queue starts as 0, 1, ..., num_blocks - 1, head first; allocation
    takes the head and evicts its cached prefix. Freed blocks with no cached
    prefix go to the head (nothing there is worth keeping).
  * A prefix hit never covers the request's last token.
  * A block whose prefix is already cached in another block stays uncached.
  * A fork shares the blocks that hold the parent's computed tokens; a write
    that starts inside a partly filled shared block first copies that block.
  * A swap-out moves the blocks holding computed tokens, in order, to the first
    free host blocks, then releases every device block as a free does; a swap-in
    takes one device block per host block from the head of the free queue and
    frees the host blocks. Copies and swaps form one ordered list of operations.
"""
from __future__ import annotations

BLOCK = 16
OP_COPY, OP_SWAP_OUT, OP_SWAP_IN = 0, 1, 2  # kinds of block operations


def ceil_blocks(tokens: int) -> int:
    return -(-tokens // BLOCK)


class Request:
    def __init__(self, tokens, salt):
        self.tokens = list(tokens)
        self.salt = salt
        self.computed = 0
        self.hashed = 0      # full blocks already offered to the cache
        self.blocks = []
        self.swapped = False
        self.host_blocks = []


class BlockPoolModel:
    """The pool as plain lists and dicts: `free` is the free queue, head at index 0."""

    def __init__(self, num_blocks: int, prefix_caching: bool, num_host_blocks: int = 0):
        if num_blocks < 1:
            raise ValueError("num_blocks must be >= 1")
        self.prefix = bool(prefix_caching)
        self.ref = [0] * num_blocks
        self.free = list(range(num_blocks))
        self.key_of = [None] * num_blocks   # prefix key a block caches, or None
        self.cache = {}                     # prefix key -> block
        self.reqs = {}
        self.ops = []                       # (kind, source, destination), in order
        self.host_free = list(range(num_host_blocks))

    # ---------------------------------------------------------------- rules
    def prefix_key(self, r: Request, i: int):
        """Identity of full block i of r: its extra key and every token up to its end."""
        return (r.salt, tuple(r.tokens[:BLOCK * (i + 1)]))

    def max_hit_blocks(self, r: Request) -> int:
        """Full blocks a hit may cover: never the block holding the last token's slot."""
        return (len(r.tokens) - 1) // BLOCK

    def requeue(self, b: int) -> None:
        """A block whose last reference went: cached ones to the tail, the rest to the head."""
        if self.key_of[b] is not None:
            self.free.append(b)
        else:
            self.free.insert(0, b)

    def release_order(self, blocks):
        """Blocks of a released request, last block first."""
        return list(reversed(blocks))

    def take_head(self) -> int:
        b = self.free.pop(0)
        if self.key_of[b] is not None:
            del self.cache[self.key_of[b]]
            self.key_of[b] = None
        self.ref[b] = 1
        return b

    def needs_copy(self, r: Request, start: int, n_new: int) -> bool:
        first = start // BLOCK
        return (n_new > 0 and start % BLOCK != 0 and first < len(r.blocks)
                and self.ref[r.blocks[first]] > 1)

    # ---------------------------------------------------------------- calls
    def add_request(self, rid, tokens, salt=0):
        if rid in self.reqs or rid < 0 or len(tokens) < 1:
            raise ValueError("bad request")
        self.reqs[rid] = Request(tokens, salt)

    def append_tokens(self, rid, tokens):
        self.reqs[rid].tokens.extend(tokens)

    def prefix_hits(self, r: Request):
        if not self.prefix or r.blocks or r.swapped:
            return []
        hits = []
        for i in range(self.max_hit_blocks(r)):
            b = self.cache.get(self.prefix_key(r, i))
            if b is None:
                break
            hits.append(b)
        return hits

    def prefix_hit_tokens(self, rid) -> int:
        return BLOCK * len(self.prefix_hits(self.reqs[rid]))

    def allocate_slots(self, rid, n_new, lookahead=0):
        """Returns the hit token count, or None when the free queue is too short.
        lookahead: positions past the request's known tokens that the step also writes
        (draft tokens of speculative decoding); the blocks cover them too."""
        r = self.reqs[rid]
        if r.swapped:
            raise ValueError("request is swapped out")
        hits = self.prefix_hits(r)
        start = r.computed + BLOCK * len(hits)
        total = start + n_new
        if n_new < 0 or lookahead < 0 or total > len(r.tokens):
            raise ValueError("allocation beyond the request's tokens")
        fresh = max(0, ceil_blocks(total + lookahead) - len(r.blocks) - len(hits))
        copy = self.needs_copy(r, start, n_new + lookahead)
        need = fresh + int(copy) + sum(1 for b in hits if self.ref[b] == 0)
        if need > len(self.free):
            return None
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            r.blocks.append(b)
        r.computed = start
        if hits:
            r.hashed = len(hits)
        if copy:
            first = start // BLOCK
            src = r.blocks[first]
            dst = self.take_head()
            self.ref[src] -= 1
            r.blocks[first] = dst
            self.ops.append((OP_COPY, src, dst))
        for _ in range(fresh):
            r.blocks.append(self.take_head())
        return BLOCK * len(hits)

    def commit(self, rid, num_computed):
        r = self.reqs[rid]
        if not r.computed <= num_computed <= min(BLOCK * len(r.blocks), len(r.tokens)):
            raise ValueError("computed count out of range")
        r.computed = num_computed
        full = num_computed // BLOCK
        if self.prefix:
            for i in range(r.hashed, full):
                b = r.blocks[i]
                key = self.prefix_key(r, i)
                if self.key_of[b] is None and key not in self.cache:
                    self.cache[key] = b
                    self.key_of[b] = key
        r.hashed = max(r.hashed, full)

    def free_request(self, rid, keep=False):
        r = self.reqs[rid]
        for b in self.release_order(r.blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.requeue(b)
        self.host_free.extend(r.host_blocks)
        if keep:
            r.blocks, r.computed, r.hashed = [], 0, 0
            r.host_blocks, r.swapped = [], False
        else:
            del self.reqs[rid]

    def swap_out(self, rid):
        """True, or False when the swap space is short (nothing changed)."""
        r = self.reqs[rid]
        if r.swapped:
            raise ValueError("already swapped out")
        keep = ceil_blocks(r.computed)
        if keep > len(self.host_free):
            return False
        for i in range(keep):
            h = self.host_free.pop(0)
            self.ops.append((OP_SWAP_OUT, r.blocks[i], h))
            r.host_blocks.append(h)
        for b in self.release_order(r.blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.requeue(b)
        r.blocks, r.hashed, r.swapped = [], 0, keep > 0
        return True

    def swap_in(self, rid):
        """True, or False when the free queue is short (nothing changed)."""
        r = self.reqs[rid]
        if not r.swapped:
            raise ValueError("not swapped out")
        if len(r.host_blocks) > len(self.free):
            return False
        for h in r.host_blocks:
            d = self.take_head()
            self.ops.append((OP_SWAP_IN, h, d))
            r.blocks.append(d)
            self.host_free.append(h)
        r.host_blocks, r.swapped, r.hashed = [], False, 0
        return True

    def fork(self, parent, child):
        if child in self.reqs or child < 0:
            raise ValueError("bad child id")
        p = self.reqs[parent]
        if p.swapped:
            raise ValueError("parent is swapped out")
        c = Request(p.tokens, p.salt)
        c.computed = p.computed
        c.hashed = min(p.hashed, p.computed // BLOCK)
        c.blocks = p.blocks[:ceil_blocks(p.computed)]
        for b in c.blocks:
            self.ref[b] += 1
        self.reqs[child] = c

    def take_ops(self):
        out, self.ops = self.ops, []
        return out

    def block_table(self, rid):
        return list(self.reqs[rid].blocks)

    def slot_mapping(self, rid, start, n):
        r = self.reqs[rid]
        if start < 0 or n < 0 or start + n > BLOCK * len(r.blocks):
            raise ValueError("positions outside the request's blocks")
        return [r.blocks[p // BLOCK] * BLOCK + p % BLOCK for p in range(start, start + n)]

    def num_cached(self) -> int:
        return sum(1 for k in self.key_of if k is not None)
