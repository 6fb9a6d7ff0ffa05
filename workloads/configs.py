"""Seeded synthetic workloads for attention over a paged KV cache.

Everything here is input preparation: request lengths, placement of 16-token
physical blocks in one pre-sized pool, per-request block tables, slot mappings
for the tokens to be written, and N(0,1) values for Q, K and V (rounded to
bfloat16 where the workload is bf16). No attention arithmetic lives here; the
oracle and the HIP path both consume these arrays unchanged.

Recipe (every workload):
  rng = numpy.random.default_rng(seed); draws happen in the order
  lengths -> placement (one rng.permutation of the pool) -> Q -> K -> V.
  Values are float32 standard normals drawn in chunks of CHUNK_VALUES, then
  rounded to bfloat16 (nearest, ties to even) for bf16 workloads.
  Each request owns ceil(L/16) blocks, taken as consecutive slices of the
  permutation (after the shared-prefix blocks, when there is a shared prefix);
  table entries past a request's last block hold one unused ("spare") block id,
  or -1 when the pool has no spare block.
  Requests are ordered prefills first, then decodes. A prefill request has n
  new tokens (its query rows); a decode request has one new token (its query).
  The K/V of every token before the new ones is written in set-up; the new
  tokens' K/V is written in the step, before attention.
  All pool slots start as quiet-NaN bit patterns, so any read of a slot that
  does not belong to a request's logical context shows up in the output.

Block size 16 and the ceil(new_tokens / 16) allocation rule are the defaults
described in the arcyou teardown of vLLM, section "PagedAttention: the KV
cache is paged, like virtual memory".
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

BLOCK_SIZE = 16
POISON_BITS = {"bf16": 0x7FC0, "f32": 0x7FC00000}
CHUNK_VALUES = 1 << 24

CONFIG_NAMES = {
    1: "tiny_decode_f32",
    2: "decode_batch_bf16",
    3: "prefix_shared_decode_bf16",
    4: "mixed_step_bf16",
    5: "long_context_decode_bf16",
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16, nearest with ties to even; return raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def blocks_needed(num_tokens) -> int:
    """Blocks a request of num_tokens occupies: ceil(num_tokens / 16)."""
    return -(-int(num_tokens) // BLOCK_SIZE)


def _normal(rng: np.random.Generator, rows: int, row_shape, dtype: str) -> np.ndarray:
    """Draw rows x row_shape standard normals (float32) in fixed-size chunks; bf16 -> uint16 bits."""
    per_row = int(np.prod(row_shape))
    out_dtype = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((rows,) + tuple(row_shape), dtype=out_dtype)
    flat = out.reshape(rows, per_row)
    chunk_rows = max(1, CHUNK_VALUES // max(per_row, 1))
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal(size=(r1 - r0, per_row), dtype=np.float32)
        flat[r0:r1] = f32_to_bf16_bits(x) if dtype == "bf16" else x
    return out


@dataclass
class PoolSpec:
    """One layer's KV pool: two tensors [num_blocks, 16, num_kv_heads, head_dim]."""
    num_blocks: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "bf16" (uint16 bit storage) or "f32" (float32 storage)
    block_size: int = BLOCK_SIZE

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def storage_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)


@dataclass
class KVWrite:
    key: np.ndarray           # [N, Hkv, D] storage dtype
    value: np.ndarray         # [N, Hkv, D]
    slot_mapping: np.ndarray  # int32 [N]; -1 = skip


@dataclass
class DecodeBatch:
    q: np.ndarray             # [S, Hq, D]
    block_tables: np.ndarray  # int32 [S, W]
    context_lens: np.ndarray  # int32 [S]

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if len(self.context_lens) else 0


@dataclass
class PrefillBatch:
    q: np.ndarray                # [T, Hq, D]
    query_start_loc: np.ndarray  # int32 [S+1]
    seq_lens: np.ndarray         # int32 [S], total KV length including this chunk
    block_tables: np.ndarray     # int32 [S, W]

    @property
    def max_query_len(self) -> int:
        return int(np.diff(self.query_start_loc).max()) if len(self.seq_lens) else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0


@dataclass
class Workload:
    name: str
    spec: PoolSpec
    scale: float
    key_tokens: np.ndarray        # [U, Hkv, D]: every distinct token, set-up tokens first
    value_tokens: np.ndarray
    slots: np.ndarray             # int32 [U]
    num_setup_tokens: int
    token_index: List[np.ndarray]  # per request: logical position -> row of key_tokens
    block_tables: np.ndarray      # int32 [R, W], prefills first
    lengths: np.ndarray           # int32 [R], KV length after the step
    new_tokens: np.ndarray        # int32 [R], tokens written in the step
    num_prefills: int
    query: np.ndarray             # [T, Hq, D]: prefill rows, then one row per decode
    shared_prefix_tokens: int = 0

    @property
    def num_requests(self) -> int:
        return len(self.lengths)

    @property
    def setup(self) -> KVWrite:
        n = self.num_setup_tokens
        return KVWrite(self.key_tokens[:n], self.value_tokens[:n], self.slots[:n])

    @property
    def step_write(self) -> KVWrite:
        n = self.num_setup_tokens
        return KVWrite(self.key_tokens[n:], self.value_tokens[n:], self.slots[n:])

    @property
    def num_prefill_rows(self) -> int:
        return int(self.new_tokens[: self.num_prefills].sum())

    @property
    def prefill(self) -> Optional[PrefillBatch]:
        if self.num_prefills == 0:
            return None
        n = self.new_tokens[: self.num_prefills]
        qsl = np.zeros(self.num_prefills + 1, dtype=np.int32)
        qsl[1:] = np.cumsum(n)
        return PrefillBatch(
            q=self.query[: self.num_prefill_rows],
            query_start_loc=qsl,
            seq_lens=self.lengths[: self.num_prefills].copy(),
            block_tables=self.block_tables[: self.num_prefills],
        )

    @property
    def decode(self) -> Optional[DecodeBatch]:
        if self.num_prefills == self.num_requests:
            return None
        return DecodeBatch(
            q=self.query[self.num_prefill_rows:],
            block_tables=self.block_tables[self.num_prefills:],
            context_lens=self.lengths[self.num_prefills:].copy(),
        )

    def logical(self, request: int):
        """K and V of a request's logical context, in storage bits, [L, Hkv, D]."""
        idx = self.token_index[request]
        return self.key_tokens[idx], self.value_tokens[idx]

    def kv_bytes_attended(self) -> int:
        """K+V bytes of the decode requests' attended tokens (logical)."""
        L = self.lengths[self.num_prefills:].astype(np.int64)
        s = self.spec
        return int(L.sum()) * 2 * s.num_kv_heads * s.head_dim * s.elem_bytes


def _assemble(name, rng, *, Hq, Hkv, D, dtype, lengths, new_tokens, num_prefills,
              shared_prefix_tokens=0, num_blocks=None, slack_tenths=1) -> Workload:
    """Place the requests in a pool, build tables and slots, then draw Q, K, V.

    lengths/new_tokens are per request (prefills first). The rng has already
    been used for the lengths; this draws placement, then Q, then K, then V.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    new_tokens = np.asarray(new_tokens, dtype=np.int64)
    R = len(lengths)
    assert np.all(lengths >= 1) and np.all(new_tokens >= 1) and np.all(new_tokens <= lengths)
    assert np.all(new_tokens[num_prefills:] == 1)
    P = int(shared_prefix_tokens)
    assert P % BLOCK_SIZE == 0
    if P:
        assert np.all(lengths - new_tokens >= P), "the shared prefix must be cached"
    prefix_blocks = P // BLOCK_SIZE
    private_blocks = np.array([blocks_needed(L) - prefix_blocks for L in lengths], dtype=np.int64)
    total = prefix_blocks + int(private_blocks.sum())
    if num_blocks is None:
        num_blocks = -(-(total * (10 + slack_tenths)) // 10)
    assert num_blocks >= total
    spec = PoolSpec(num_blocks=int(num_blocks), num_q_heads=Hq, num_kv_heads=Hkv,
                    head_dim=D, dtype=dtype)

    # placement
    perm = rng.permutation(num_blocks).astype(np.int32)
    spare = int(perm[total]) if num_blocks > total else -1
    W = int(max(prefix_blocks + private_blocks.max(), 1)) if R else 1
    tables = np.full((R, W), spare, dtype=np.int32)
    off = prefix_blocks
    for r in range(R):
        nb = int(private_blocks[r])
        tables[r, :prefix_blocks] = perm[:prefix_blocks]
        tables[r, prefix_blocks:prefix_blocks + nb] = perm[off:off + nb]
        off += nb

    # distinct tokens: shared prefix, each request's private cached tokens, then new tokens
    rows_T = int(new_tokens[:num_prefills].sum()) + (R - num_prefills)
    token_index = [np.empty(int(L), dtype=np.int64) for L in lengths]
    slots = []
    u = 0
    if P:
        pos = np.arange(P)
        s = tables[0][pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + pos % BLOCK_SIZE
        slots.append(s)
        for r in range(R):
            token_index[r][:P] = np.arange(P)
        u = P
    for r in range(R):
        pos = np.arange(P, lengths[r] - new_tokens[r])
        slots.append(tables[r][pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + pos % BLOCK_SIZE)
        token_index[r][P:lengths[r] - new_tokens[r]] = u + np.arange(len(pos))
        u += len(pos)
    num_setup = u
    for r in range(R):
        pos = np.arange(lengths[r] - new_tokens[r], lengths[r])
        slots.append(tables[r][pos // BLOCK_SIZE].astype(np.int64) * BLOCK_SIZE + pos % BLOCK_SIZE)
        token_index[r][lengths[r] - new_tokens[r]:] = u + np.arange(len(pos))
        u += len(pos)
    slots = np.concatenate(slots).astype(np.int32) if slots else np.zeros(0, np.int32)

    q = _normal(rng, rows_T, (Hq, D), dtype)
    k = _normal(rng, u, (Hkv, D), dtype)
    v = _normal(rng, u, (Hkv, D), dtype)
    return Workload(
        name=name, spec=spec, scale=1.0 / math.sqrt(D),
        key_tokens=k, value_tokens=v, slots=slots, num_setup_tokens=num_setup,
        token_index=token_index, block_tables=tables,
        lengths=lengths.astype(np.int32), new_tokens=new_tokens.astype(np.int32),
        num_prefills=num_prefills, query=q, shared_prefix_tokens=P,
    )


def c1_tiny_decode(seed: int = 1) -> Workload:
    """4 decode requests, contexts {1,17,48,100}, 8 q / 8 kv heads, head_dim 64, fp32, pool of 64 blocks."""
    rng = np.random.default_rng(seed)
    lengths = [1, 17, 48, 100]
    return _assemble(CONFIG_NAMES[1], rng, Hq=8, Hkv=8, D=64, dtype="f32",
                     lengths=lengths, new_tokens=[1] * 4, num_prefills=0, num_blocks=64)


def c2_decode_batch(seed: int = 2, num_seqs: int = 64, len_lo: int = 512, len_hi: int = 4096,
                    Hq: int = 32, Hkv: int = 8, D: int = 128, dtype: str = "bf16") -> Workload:
    """Decode batch: lengths uniform in [len_lo, len_hi]; pool = needed blocks + 10%, random placement."""
    rng = np.random.default_rng(seed)
    lengths = rng.integers(len_lo, len_hi + 1, size=num_seqs)
    return _assemble(CONFIG_NAMES[2], rng, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     lengths=lengths, new_tokens=np.ones(num_seqs, np.int64), num_prefills=0)


def c3_prefix_shared(seed: int = 3, num_seqs: int = 256, prefix_tokens: int = 2048,
                     tail_lo: int = 64, tail_hi: int = 512, Hq: int = 32, Hkv: int = 8,
                     D: int = 128, dtype: str = "bf16") -> Workload:
    """Decode requests sharing one cached prefix (same physical blocks) plus private tails."""
    rng = np.random.default_rng(seed)
    tails = rng.integers(tail_lo, tail_hi + 1, size=num_seqs)
    lengths = prefix_tokens + tails
    return _assemble(CONFIG_NAMES[3], rng, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     lengths=lengths, new_tokens=np.ones(num_seqs, np.int64), num_prefills=0,
                     shared_prefix_tokens=prefix_tokens)


def c4_mixed_step(seed: int = 4, num_prefills: int = 4, new_tokens: int = 1536,
                  cached_lo: int = 0, cached_hi: int = 4096, num_decodes: int = 96,
                  dec_lo: int = 1024, dec_hi: int = 8192, cached=None, Hq: int = 32,
                  Hkv: int = 8, D: int = 128, dtype: str = "bf16") -> Workload:
    """One continuous-batching step: chunked prefills over cached tokens, plus decodes."""
    rng = np.random.default_rng(seed)
    c = rng.integers(cached_lo, cached_hi + 1, size=num_prefills)
    if cached is not None:
        c = np.asarray(cached, dtype=np.int64)
        assert len(c) == num_prefills
    dec = rng.integers(dec_lo, dec_hi + 1, size=num_decodes)
    lengths = np.concatenate([c + new_tokens, dec])
    new = np.concatenate([np.full(num_prefills, new_tokens), np.ones(num_decodes, np.int64)])
    return _assemble(CONFIG_NAMES[4], rng, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     lengths=lengths, new_tokens=new, num_prefills=num_prefills)


def c5_long_decode(seed: int = 5, num_seqs: int = 8, length: int = 131072, Hq: int = 64,
                   Hkv: int = 8, D: int = 128, dtype: str = "bf16", num_blocks=None) -> Workload:
    """Long-context decode; by default the pool holds exactly the blocks in use."""
    rng = np.random.default_rng(seed)
    lengths = np.full(num_seqs, length, dtype=np.int64)
    if num_blocks is None:
        num_blocks = num_seqs * blocks_needed(length)
    return _assemble(CONFIG_NAMES[5], rng, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype,
                     lengths=lengths, new_tokens=np.ones(num_seqs, np.int64), num_prefills=0,
                     num_blocks=num_blocks)


def custom_decode(seed: int, lengths, Hq: int, Hkv: int, D: int, dtype: str,
                  shared_prefix_tokens: int = 0, num_blocks=None, slack_tenths: int = 1) -> Workload:
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    return _assemble("custom_decode", rng, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, lengths=lengths,
                     new_tokens=np.ones(len(lengths), np.int64), num_prefills=0,
                     shared_prefix_tokens=shared_prefix_tokens, num_blocks=num_blocks,
                     slack_tenths=slack_tenths)


def custom_prefill(seed: int, cached, new, Hq: int, Hkv: int, D: int, dtype: str,
                   decode_lengths=(), num_blocks=None) -> Workload:
    """Chunked prefills (cached[i] tokens already in the pool, new[i] in the chunk), then decodes."""
    rng = np.random.default_rng(seed)
    cached = np.asarray(cached, dtype=np.int64)
    new = np.asarray(new, dtype=np.int64)
    dec = np.asarray(decode_lengths, dtype=np.int64)
    lengths = np.concatenate([cached + new, dec])
    nt = np.concatenate([new, np.ones(len(dec), np.int64)])
    return _assemble("custom_prefill", rng, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, lengths=lengths,
                     new_tokens=nt, num_prefills=len(cached), num_blocks=num_blocks)


_BUILDERS = {1: c1_tiny_decode, 2: c2_decode_batch, 3: c3_prefix_shared, 4: c4_mixed_step,
             5: c5_long_decode}


def make(index: int, seed: Optional[int] = None, **overrides) -> Workload:
    """Workload for config index 1..5 (seed defaults to the index)."""
    return _BUILDERS[index](seed=index if seed is None else seed, **overrides)
