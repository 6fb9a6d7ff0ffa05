"""Plain, slow CPU oracle for attention over a paged KV cache (numpy, float64).

TEST INFRASTRUCTURE. Only the tests, the smoke check in __graft_entry__ and the
benchmark's CPU-baseline leg may import, call or run this module. The HIP
library and its Python binding never import it, and it imports nothing from
them: the two share no code, constants or helpers.

What the method computes, and where each step comes from:
  * KV memory is one pool of fixed-size blocks, 16 tokens each; a request holds
    a list of physical block ids, and attention is handed a per-request block
    table that maps logical token positions to physical blocks and gathers K/V
    from wherever those blocks live (arcyou teardown of vLLM paged attention,
    section "PagedAttention: the KV cache is paged, like virtual memory").
  * The logical context is contiguous even though the physical pages are not
    (kenhuang vLLM course, "Introduction", section "PagedAttention (intuition)").
    Paging is therefore only a storage scheme: the result is exactly ordinary
    scaled dot-product attention over each request's logical context, which is
    what this oracle writes out. That formula, softmax(q K^T / sqrt(d)) V, is
    not printed on the pages; it is the standard definition they take as given.
  * The KV cache grows one token at a time, and every new token reads all past
    K/V (arcyou teardown, "The problem both ideas solve"; kenhuang,
    "PagedAttention (intuition)"): new K/V is written into slots, then attended.
  * Prefill and decode are the same kind of work, and a long prompt may be split
    across steps (arcyou teardown, section "Continuous batching: rebuild the
    batch every step"): a chunk of n new tokens continues after the tokens
    already cached.
  * Prefix sharing maps several requests onto the same physical blocks with no
    copy (arcyou teardown, "PagedAttention" section, prefix sharing paragraph).

Readings taken where the pages are silent:
  * Pool layout: two tensors (K and V), each [num_blocks, 16, kv_heads, head_dim].
  * A slot is block_id * 16 + offset; slot -1 means "write nothing".
  * Grouped-query attention: query head h reads kv head h // (q_heads / kv_heads).
  * Scale is 1 / sqrt(head_dim).
  * A decode request's context length counts every token it attends, including
    its own newest token, whose K/V is written before attention.
  * Chunked prefill is aligned bottom-right: row i of an n-row chunk over a
    context of L tokens attends keys 0 .. L - n + i.
  * A context of length 0 is an error (softmax over nothing is undefined).

Every function works on raw storage bits (bf16 as uint16, fp32 as float32) for
the pool and decodes to float64 exactly before any arithmetic.
"""
from __future__ import annotations

import numpy as np

BLOCK_SIZE = 16


# ----------------------------------------------------------------------------- storage
def to_float64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored elements (bf16: the upper half of an IEEE float32)."""
    if dtype == "bf16":
        wide = bits.astype(np.uint32) << np.uint32(16)
        return wide.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(bits, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def empty_pool(num_blocks: int, num_kv_heads: int, head_dim: int, dtype: str, fill_bits: int):
    """A pool tensor [num_blocks, 16, kv_heads, head_dim] whose every element holds fill_bits."""
    if dtype == "bf16":
        return np.full((num_blocks, BLOCK_SIZE, num_kv_heads, head_dim), fill_bits, dtype=np.uint16)
    word = np.array([fill_bits], dtype=np.uint32).view(np.float32)[0]
    return np.full((num_blocks, BLOCK_SIZE, num_kv_heads, head_dim), word, dtype=np.float32)


def slot_location(slot: int):
    """Physical (block id, offset in block) of a flat slot."""
    return divmod(int(slot), BLOCK_SIZE)


def write_kv(k_pool, v_pool, key, value, slot_mapping) -> None:
    """Copy each new token's K and V rows, unchanged, into its slot (in place).

    Tokens whose slot is -1 are skipped. Slots must be distinct and in range.
    """
    num_slots = k_pool.shape[0] * BLOCK_SIZE
    taken = set()
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot == -1:
            continue
        if not 0 <= slot < num_slots:
            raise IndexError(f"slot {slot} of token {i} is outside the pool")
        if slot in taken:
            raise ValueError(f"slot {slot} written twice")
        taken.add(slot)
        b, o = slot_location(slot)
        k_pool[b, o] = key[i]
        v_pool[b, o] = value[i]


def copy_blocks(k_pool, v_pool, block_pairs) -> None:
    """Duplicate whole blocks in place, K and V: block dst becomes a bit copy of block src.

    This is the copy-on-write step for forked sequences that share blocks until
    one writes into a shared block (aitrending, "The 1960s Operating System Trick
    That Makes vLLM 4x Faster", Technical Details). Destinations must be distinct
    and no block may be both a source and a destination in one call.
    """
    pairs = np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2)
    src, dst = pairs[:, 0].tolist(), pairs[:, 1].tolist()
    if len(set(dst)) != len(dst):
        raise ValueError("a block is a destination twice")
    if set(dst) & set(src):
        raise ValueError("a block is both a source and a destination")
    nb = k_pool.shape[0]
    for a, b in zip(src, dst):
        if not (0 <= a < nb and 0 <= b < nb):
            raise IndexError("block pair outside the pool")
        k_pool[b] = k_pool[a]
        v_pool[b] = v_pool[a]


def swap_blocks(k_pool, v_pool, host_k, host_v, block_pairs, to_host: bool) -> None:
    """Move whole blocks between the device pool and a host swap pool, K and V alike.

    Preemption may keep a request's K/V by swapping its blocks to CPU memory
    instead of recomputing them (aitrending, "The 1960s Operating System Trick
    That Makes vLLM 4x Faster", Technical Details). to_host: pairs are
    (device block, host block); otherwise (host block, device block).
    Destinations must be distinct.
    """
    pairs = np.asarray(block_pairs, dtype=np.int64).reshape(-1, 2)
    dst = pairs[:, 1].tolist()
    if len(set(dst)) != len(dst):
        raise ValueError("a block is a destination twice")
    for a, b in pairs.tolist():
        dev, hst = (a, b) if to_host else (b, a)
        if not (0 <= dev < k_pool.shape[0] and 0 <= hst < host_k.shape[0]):
            raise IndexError("block pair outside a pool")
        if to_host:
            host_k[hst] = k_pool[dev]
            host_v[hst] = v_pool[dev]
        else:
            k_pool[dev] = host_k[hst]
            v_pool[dev] = host_v[hst]


def blocks_for(num_tokens: int) -> int:
    """Blocks covering num_tokens tokens: ceil(num_tokens / 16)."""
    return (int(num_tokens) + BLOCK_SIZE - 1) // BLOCK_SIZE


def gather_logical(pool, table_row, length: int):
    """A request's first `length` tokens in logical order, read through its block table (bits)."""
    nb = blocks_for(length)
    ids = np.asarray(table_row[:nb], dtype=np.int64)
    if nb and (ids.min() < 0 or ids.max() >= pool.shape[0]):
        raise IndexError("block table entry outside the pool")
    rows = pool[ids].reshape((nb * BLOCK_SIZE,) + pool.shape[2:])
    return rows[:length]


# ----------------------------------------------------------------------------- attention
def kv_head_of(q_head: int, group: int) -> int:
    """kv head read by a query head under grouped-query attention."""
    return q_head // group


def last_key(row: int, num_rows: int, context_len: int) -> int:
    """Last key position visible to row `row` of a chunk of num_rows new tokens ending the context."""
    return context_len - num_rows + row


def softmax_weights(scores: np.ndarray) -> np.ndarray:
    """Row-wise softmax; -inf scores get weight 0."""
    m = np.max(scores, axis=-1, keepdims=True)
    w = np.exp(scores - m)
    return w / np.sum(w, axis=-1, keepdims=True)


def attend(q_rows, keys, values, limits, scale):
    """softmax(scale * q K^T) V with row i restricted to keys 0..limits[i] (all float64)."""
    scores = scale * (q_rows @ keys.T)
    hidden = np.arange(keys.shape[0])[None, :] > np.asarray(limits)[:, None]
    scores = np.where(hidden, -np.inf, scores)
    return softmax_weights(scores) @ values


def _checked_group(q_heads: int, kv_heads: int) -> int:
    if q_heads % kv_heads:
        raise ValueError("q heads must be a multiple of kv heads")
    return q_heads // kv_heads


def default_scale(head_dim: int) -> float:
    return 1.0 / np.sqrt(float(head_dim))


def decode(q, k_pool, v_pool, block_tables, context_lens, dtype, scale=None, pairs=None):
    """Decode attention: one query per request at its last position, over all its context.

    q [S, Hq, D] (storage bits); returns float64 [S, Hq, D]. With `pairs`, a list
    of (request, q head), only those rows are computed (others stay NaN).
    """
    S, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    G = _checked_group(Hq, Hkv)
    scale = default_scale(D) if scale is None else scale
    out = np.full((S, Hq, D), np.nan)
    todo = {}
    for s, h in (pairs if pairs is not None else [(s, h) for s in range(S) for h in range(Hq)]):
        todo.setdefault(int(s), set()).add(int(h))
    for s, heads in sorted(todo.items()):
        L = int(context_lens[s])
        if L < 1:
            raise ValueError("context length must be at least 1")
        kb = gather_logical(k_pool, block_tables[s], L)
        vb = gather_logical(v_pool, block_tables[s], L)
        by_kv = {}
        for h in sorted(heads):
            by_kv.setdefault(kv_head_of(h, G), []).append(h)
        for j, hs in by_kv.items():
            K = to_float64(kb[:, j], dtype)
            V = to_float64(vb[:, j], dtype)
            Q = to_float64(q[s, hs], dtype)
            limits = [last_key(0, 1, L)] * len(hs)
            out[s, hs] = attend(Q, K, V, limits, scale)
    return out


def prefill_chunk(q, k_pool, v_pool, query_start_loc, seq_lens, block_tables, dtype, scale=None):
    """Causal attention for each request's chunk of new tokens over its cached + new context.

    q [T, Hq, D] (storage bits), rows of request s are query_start_loc[s]:query_start_loc[s+1];
    seq_lens[s] is the request's total context including the chunk. Returns float64 [T, Hq, D].
    """
    T, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    G = _checked_group(Hq, Hkv)
    scale = default_scale(D) if scale is None else scale
    out = np.full((T, Hq, D), np.nan)
    for s in range(len(seq_lens)):
        a, b = int(query_start_loc[s]), int(query_start_loc[s + 1])
        n, L = b - a, int(seq_lens[s])
        if n == 0:
            continue
        if L < n:
            raise ValueError("a chunk cannot be longer than its context")
        kb = gather_logical(k_pool, block_tables[s], L)
        vb = gather_logical(v_pool, block_tables[s], L)
        limits = [last_key(i, n, L) for i in range(n)]
        for j in range(Hkv):
            K = to_float64(kb[:, j], dtype)
            V = to_float64(vb[:, j], dtype)
            for h in range(Hq):
                if kv_head_of(h, G) != j:
                    continue
                out[a:b, h] = attend(to_float64(q[a:b, h], dtype), K, V, limits, scale)
    return out


def split_kv_decode(q, k_pool, v_pool, block_tables, context_lens, dtype, partition_tokens,
                    scale=None):
    """Decode computed partition by partition and merged, as a split-KV kernel does.

    Each partition of `partition_tokens` keys yields (m, l, acc) = (max score,
    sum of exp(score - m), sum of exp(score - m) * v); the merge rescales every
    partition to the global maximum M and returns sum(e^(m-M) acc) / sum(e^(m-M) l).
    Algebraically identical to decode(); kept to pin that identity.
    """
    S, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    G = _checked_group(Hq, Hkv)
    scale = default_scale(D) if scale is None else scale
    out = np.empty((S, Hq, D))
    for s in range(S):
        L = int(context_lens[s])
        K = to_float64(gather_logical(k_pool, block_tables[s], L), dtype)
        V = to_float64(gather_logical(v_pool, block_tables[s], L), dtype)
        for h in range(Hq):
            j = kv_head_of(h, G)
            qv = to_float64(q[s, h], dtype)
            parts = []
            for p0 in range(0, L, partition_tokens):
                sc = scale * (K[p0:p0 + partition_tokens, j] @ qv)
                m = sc.max()
                e = np.exp(sc - m)
                parts.append((m, e.sum(), e @ V[p0:p0 + partition_tokens, j]))
            M = max(m for m, _, _ in parts)
            num = sum(np.exp(m - M) * acc for m, _, acc in parts)
            den = sum(np.exp(m - M) * l for m, l, _ in parts)
            out[s, h] = num / den
    return out


def gather_kv(pool, block_tables, context_lens):
    """Each request's logical K (or V) rows as stored bits: list of [L, Hkv, D]."""
    return [gather_logical(pool, block_tables[s], int(context_lens[s])).copy()
            for s in range(len(context_lens))]
