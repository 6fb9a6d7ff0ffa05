"""Pins for the fp64 oracle, independent of the oracle's own formulas (CPU only).

Each pin ties the oracle to something outside itself: torch's scaled-dot-product
attention on contiguous K/V (a library routine), closed forms, exact special
cases, and invariants the pages state (a request's logical context is
contiguous while its physical blocks need not be; shared prefix blocks are used
with no copy; a chunk continues after the cached tokens). The planted-mistake
test at the end checks that each plausible slip in the oracle trips a pin.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
from oracle import paged_attention as pa_oracle
import workloads
from workloads import POISON_BITS, custom_decode, custom_prefill
from oracle_support import oracle_pools, oracle_decode, oracle_prefill, values64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- references
def sdpa_rows(q64, k64, v64, causal):
    """torch SDPA on contiguous K/V: q [n, Hq, D], k/v [L, Hkv, D] float64 (default scale)."""
    q = torch.from_numpy(q64).permute(1, 0, 2)[None]
    k = torch.from_numpy(k64).permute(1, 0, 2)[None]
    v = torch.from_numpy(v64).permute(1, 0, 2)[None]
    o = F.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=True)
    return o[0].permute(1, 0, 2).numpy()


def logical64(w, r):
    kb, vb = w.logical(r)
    return values64(kb, w.spec.dtype), values64(vb, w.spec.dtype)


# ----------------------------------------------------------------------------- pins
def pin_storage_decode():
    """bf16/fp32 storage bits decode to the exact IEEE values."""
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F80, 0x8000, 0x4049], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, math.inf, -0.0, 3.140625]
    got = oracle.to_float64(bits, "bf16")
    assert got.tolist() == want
    assert np.signbit(got[5])
    f = np.array([0.1, -3.5, 1e-40], dtype=np.float32)
    assert oracle.to_float64(f, "f32").tolist() == [float(x) for x in f]


def pin_write_slots():
    """Slot s lands in block s // 16 at offset s % 16; -1 writes nothing; others untouched."""
    k = oracle.empty_pool(4, 2, 3, "bf16", 0x7FC0)
    v = oracle.empty_pool(4, 2, 3, "bf16", 0x7FC0)
    key = np.arange(3 * 2 * 3, dtype=np.uint16).reshape(3, 2, 3) + 100
    val = key + 1000
    oracle.write_kv(k, v, key, val, np.array([37, -1, 0], dtype=np.int32))
    assert np.array_equal(k[2, 5], key[0]) and np.array_equal(v[2, 5], val[0])
    assert np.array_equal(k[0, 0], key[2]) and np.array_equal(v[0, 0], val[2])
    touched = np.zeros((4, 16), bool)
    touched[2, 5] = touched[0, 0] = True
    assert np.all(k[~touched] == 0x7FC0) and np.all(v[~touched] == 0x7FC0)


def pin_roundtrip(seed=11):
    """gather(write(x)) == x bit for bit, through the workload's random placement."""
    w = custom_decode(seed, [1, 16, 17, 40], Hq=4, Hkv=2, D=8, dtype="bf16")
    k, v = oracle_pools(w)
    d = w.decode
    gk = oracle.gather_kv(k, d.block_tables, d.context_lens)
    gv = oracle.gather_kv(v, d.block_tables, d.context_lens)
    for r in range(w.num_requests):
        lk, lv = w.logical(r)
        assert np.array_equal(gk[r], lk) and np.array_equal(gv[r], lv)


def pin_decode_vs_sdpa(seed=3, lengths=(1, 5, 16, 33, 70), Hq=8, Hkv=4, D=16, dtype="bf16"):
    """Paged decode equals torch SDPA on the contiguous logical context (GQA, default scale)."""
    w = custom_decode(seed, list(lengths), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    k, v = oracle_pools(w)
    got = oracle_decode(w, k, v)
    q64 = values64(w.decode.q, dtype)
    for r in range(w.num_requests):
        K, V = logical64(w, r)
        ref = sdpa_rows(q64[r:r + 1], K, V, causal=False)[0]
        assert np.max(np.abs(got[r] - ref)) <= 1e-12, r


def pin_prefill_vs_sdpa(seed=5, cached=(0, 3, 16, 21), new=(7, 1, 16, 29), Hq=4, Hkv=2, D=8,
                        dtype="bf16"):
    """A chunk's rows equal the last rows of full causal attention over cached + new tokens."""
    w = custom_prefill(seed, list(cached), list(new), Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    k, v = oracle_pools(w)
    got = oracle_prefill(w, k, v)
    p = w.prefill
    for r in range(len(cached)):
        a, b = p.query_start_loc[r], p.query_start_loc[r + 1]
        K, V = logical64(w, r)
        L = K.shape[0]
        # full causal over all L tokens needs queries for the cached positions too: use
        # zeros there (their rows are discarded); SDPA's causal mask is unambiguous at Lq == Lk.
        qfull = np.zeros((L, Hq, D))
        qfull[L - (b - a):] = values64(p.q[a:b], dtype)
        ref = sdpa_rows(qfull, K, V, causal=True)[L - (b - a):]
        assert np.max(np.abs(got[a:b] - ref)) <= 1e-12, r


def pin_context_one():
    """A context of one token returns that token's V exactly."""
    w = custom_decode(7, [1, 1, 1], Hq=4, Hkv=2, D=8, dtype="bf16")
    k, v = oracle_pools(w)
    got = oracle_decode(w, k, v)
    for r in range(3):
        _, V = logical64(w, r)
        for h in range(4):
            assert np.array_equal(got[r, h], V[0, h // 2])


def pin_zero_query_mean():
    """q = 0 gives every key the weight 1/L: the output is the mean of the V rows."""
    w = custom_decode(9, [1, 7, 40], Hq=2, Hkv=1, D=8, dtype="f32")
    w.query[:] = 0
    k, v = oracle_pools(w)
    got = oracle_decode(w, k, v)
    for r in range(3):
        _, V = logical64(w, r)
        assert np.max(np.abs(got[r] - V[:, 0].mean(axis=0))) <= 1e-12


def pin_one_hot():
    """A key equal to alpha*q dominates: the output tends to that key's V."""
    w = custom_decode(13, [40], Hq=1, Hkv=1, D=8, dtype="f32")
    d = w.decode
    q = np.zeros(8, np.float32)
    q[2] = 1.0
    w.query[0, 0] = q
    kb = w.key_tokens
    idx = w.token_index[0]
    kb[idx, 0] = 0.0
    kb[idx[23], 0] = 400.0 * q  # score 400/sqrt(8) above the others
    k, v = oracle_pools(w)
    got = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "f32")
    _, V = logical64(w, 0)
    assert np.max(np.abs(got[0, 0] - V[23, 0])) <= 1e-12


def pin_two_key_closed_form():
    """Two keys: the weights are a logistic function of the score gap."""
    k = oracle.empty_pool(2, 1, 2, "f32", 0x7FC00000)
    v = oracle.empty_pool(2, 1, 2, "f32", 0x7FC00000)
    key = np.array([[[1.0, 0.0]], [[0.0, 0.0]]], np.float32)
    val = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], np.float32)
    oracle.write_kv(k, v, key, val, np.array([16, 17], np.int32))  # block 1, offsets 0 and 1
    q = np.array([[[1.0, 0.0]]], np.float32)
    got = oracle.decode(q, k, v, np.array([[1]], np.int32), np.array([2], np.int32), "f32")
    w1 = 1.0 / (1.0 + math.exp(-1.0 / math.sqrt(2.0)))
    assert abs(got[0, 0, 0] - w1) <= 1e-15 and abs(got[0, 0, 1] - (1 - w1)) <= 1e-15


def pin_softmax_weights():
    rng = np.random.default_rng(0)
    s = rng.standard_normal((5, 37)) * 4
    s[:, 30:] = -np.inf
    w = oracle.softmax_weights(s)
    assert np.all(w >= 0) and np.all(w <= 1)
    assert np.max(np.abs(w.sum(-1) - 1)) <= 1e-12
    assert np.all(w[:, 30:] == 0)


def pin_permutation_invariance(seed=17):
    """Relabelling physical blocks (pool and tables together) leaves the output bit-identical."""
    w = custom_decode(seed, [3, 16, 50, 61], Hq=4, Hkv=2, D=8, dtype="bf16")
    k, v = oracle_pools(w)
    d = w.decode
    base = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "bf16")
    perm = np.random.default_rng(seed).permutation(k.shape[0])  # new id of old block b is perm[b]
    k2, v2 = np.empty_like(k), np.empty_like(v)
    k2[perm], v2[perm] = k, v
    bt = d.block_tables.copy()
    ok = bt >= 0
    bt[ok] = perm[bt[ok]]
    again = oracle.decode(d.q, k2, v2, bt, d.context_lens, "bf16")
    assert np.array_equal(base, again)


def pin_prefix_sharing():
    """Reading a shared prefix gives bit-identical output to reading private copies of it."""
    w = custom_decode(19, [40, 57, 33], Hq=4, Hkv=2, D=8, dtype="bf16", shared_prefix_tokens=32)
    k, v = oracle_pools(w)
    d = w.decode
    shared = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "bf16")
    assert len({tuple(d.block_tables[r, :2]) for r in range(3)}) == 1  # really shared
    # give requests 1 and 2 private copies of the two prefix blocks, in fresh blocks
    NB = k.shape[0]
    k2 = np.concatenate([k, k[d.block_tables[0, :2]], k[d.block_tables[0, :2]]])
    v2 = np.concatenate([v, v[d.block_tables[0, :2]], v[d.block_tables[0, :2]]])
    bt = d.block_tables.copy()
    bt[1, :2] = [NB, NB + 1]
    bt[2, :2] = [NB + 2, NB + 3]
    private = oracle.decode(d.q, k2, v2, bt, d.context_lens, "bf16")
    assert np.array_equal(shared, private)


def pin_gqa_equals_repeated_mha():
    """GQA with group G equals MHA whose kv heads are the GQA kv heads repeated G times."""
    w = custom_decode(23, [9, 33], Hq=8, Hkv=2, D=8, dtype="f32")
    k, v = oracle_pools(w)
    d = w.decode
    gqa = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "f32")
    mha = oracle.decode(d.q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2),
                        d.block_tables, d.context_lens, "f32")
    assert np.max(np.abs(gqa - mha)) <= 1e-13  # batched vs per-head BLAS rounding only


def pin_chunk_is_rows_of_full():
    """A chunk over c cached tokens equals rows c.. of the whole prompt prefilled at once."""
    full = custom_prefill(29, [0], [45], Hq=4, Hkv=2, D=8, dtype="bf16")
    k, v = oracle_pools(full)
    p = full.prefill
    whole = oracle_prefill(full, k, v)
    for c in (1, 16, 30, 44):
        qsl = np.array([0, 45 - c], np.int32)
        part = oracle.prefill_chunk(p.q[c:], k, v, qsl, p.seq_lens, p.block_tables, "bf16")
        assert np.max(np.abs(part - whole[c:])) <= 1e-12


def pin_decode_is_one_row_chunk():
    w = custom_decode(31, [1, 30, 64], Hq=4, Hkv=1, D=8, dtype="bf16")
    k, v = oracle_pools(w)
    d = w.decode
    dec = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "bf16")
    qsl = np.arange(4, dtype=np.int32)
    pre = oracle.prefill_chunk(d.q, k, v, qsl, d.context_lens, d.block_tables, "bf16")
    assert np.max(np.abs(dec - pre)) <= 1e-12


def pin_split_kv_identity():
    w = custom_decode(37, [1, 15, 16, 17, 100, 513], Hq=4, Hkv=2, D=8, dtype="bf16")
    k, v = oracle_pools(w)
    d = w.decode
    ref = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "bf16")
    for part in (16, 48, 256, 1024):
        got = oracle.split_kv_decode(d.q, k, v, d.block_tables, d.context_lens, "bf16", part)
        assert np.max(np.abs(got - ref)) <= 1e-12, part


def pin_copy_blocks():
    """A copied block equals its source bit for bit; nothing else changes; bad pairs raise."""
    k = oracle.empty_pool(6, 2, 4, "bf16", 0x7FC0)
    rng = np.random.default_rng(3)
    k[:] = rng.integers(0, 1 << 16, size=k.shape, dtype=np.uint16)
    v = k ^ np.uint16(0x5555)
    k0, v0 = k.copy(), v.copy()
    pa_oracle.copy_blocks(k, v, [[1, 4], [1, 5], [2, 0]])
    assert np.array_equal(k[4], k0[1]) and np.array_equal(k[5], k0[1]) and np.array_equal(k[0], k0[2])
    assert np.array_equal(v[4], v0[1]) and np.array_equal(v[0], v0[2])
    assert np.array_equal(k[[1, 2, 3]], k0[[1, 2, 3]])
    for bad in ([[1, 3], [2, 3]], [[1, 3], [3, 4]], [[1, 6]]):
        with pytest.raises((ValueError, IndexError)):
            pa_oracle.copy_blocks(k.copy(), v.copy(), bad)


def pin_copy_on_write_fork():
    """Fork a request, copy its last shared block, write the fork's next token into the copy:
    the parent's output is unchanged and the fork attends parent tokens + its new token."""
    w = custom_decode(43, [37], Hq=4, Hkv=2, D=8, dtype="bf16")
    k, v = oracle_pools(w)
    d = w.decode
    parent = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "bf16")
    spare = [b for b in range(k.shape[0]) if b not in set(d.block_tables[0, :3].tolist())][0]
    fork = d.block_tables[:1].copy()
    last = int(fork[0, 2])  # tokens 32..36 live in the third block
    pa_oracle.copy_blocks(k, v, [[last, spare]])
    fork[0, 2] = spare
    new_k = (np.arange(2 * 8, dtype=np.uint16).reshape(1, 2, 8) + 0x3F00).astype(np.uint16)
    new_v = new_k ^ np.uint16(0x0101)
    oracle.write_kv(k, v, new_k, new_v, np.array([spare * 16 + 5], np.int32))  # token 37
    again = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "bf16")
    assert np.array_equal(again, parent)
    K, V = logical64(w, 0)
    K = np.concatenate([K, values64(new_k, "bf16")])
    V = np.concatenate([V, values64(new_v, "bf16")])
    got = oracle.decode(d.q, k, v, fork, np.array([38], np.int32), "bf16")
    ref = sdpa_rows(values64(d.q, "bf16"), K, V, causal=False)
    assert np.max(np.abs(got[0] - ref[0])) <= 1e-12


def pin_swap_round_trip():
    """Blocks swapped out land bit-exact in the host pool; swapped back into other device
    blocks, a request reads the same logical context through its new table (the decode
    result is identical), and no other block changes."""
    w = custom_decode(47, [40, 9], Hq=4, Hkv=2, D=8, dtype="bf16", num_blocks=12)
    k, v = oracle_pools(w)
    d = w.decode
    before = oracle.decode(d.q, k, v, d.block_tables, d.context_lens, "bf16")
    table = d.block_tables[0, :3].tolist()
    hk = oracle.empty_pool(5, 2, 8, "bf16", 0)
    hv = hk.copy()
    k0, v0 = k.copy(), v.copy()
    pa_oracle.swap_blocks(k, v, hk, hv, [[b, h] for b, h in zip(table, (4, 0, 2))], True)
    assert np.array_equal(k, k0) and np.array_equal(v, v0)
    assert np.array_equal(hk[[4, 0, 2]], k0[table]) and np.array_equal(hv[[4, 0, 2]], v0[table])
    assert not hk[[1, 3]].any() and not hv[[1, 3]].any()
    used = set(d.block_tables.ravel().tolist())
    fresh = [b for b in range(k.shape[0]) if b not in used][:3]
    assert len(fresh) == 3
    k[table] = 0x7FC0  # the old blocks are handed to someone else
    v[table] = 0x7FC0
    k1, v1 = k.copy(), v.copy()
    pa_oracle.swap_blocks(k, v, hk, hv, [[h, b] for h, b in zip((4, 0, 2), fresh)], False)
    assert np.array_equal(k[fresh], k0[table]) and np.array_equal(v[fresh], v0[table])
    others = [b for b in range(k.shape[0]) if b not in fresh]
    assert np.array_equal(k[others], k1[others]) and np.array_equal(v[others], v1[others])
    tables = d.block_tables.copy()
    tables[0, :3] = fresh
    after = oracle.decode(d.q, k, v, tables, d.context_lens, "bf16", pairs=[(0, h) for h in range(4)])
    assert np.array_equal(after[0], before[0])
    with pytest.raises((ValueError, IndexError)):
        pa_oracle.swap_blocks(k, v, hk, hv, [[0, 1], [2, 1]], True)
    with pytest.raises((ValueError, IndexError)):
        pa_oracle.swap_blocks(k, v, hk, hv, [[0, 5]], True)


def pin_empty_context_rejected():
    k = oracle.empty_pool(2, 1, 4, "f32", 0)
    with pytest.raises(ValueError):
        oracle.decode(np.zeros((1, 1, 4), np.float32), k, k, np.zeros((1, 1), np.int32),
                      np.zeros(1, np.int32), "f32")


ALL_PINS = [
    pin_storage_decode, pin_write_slots, pin_roundtrip, pin_decode_vs_sdpa, pin_prefill_vs_sdpa,
    pin_context_one, pin_zero_query_mean, pin_one_hot, pin_two_key_closed_form,
    pin_softmax_weights, pin_permutation_invariance, pin_prefix_sharing,
    pin_gqa_equals_repeated_mha, pin_chunk_is_rows_of_full, pin_decode_is_one_row_chunk,
    pin_split_kv_identity, pin_empty_context_rejected, pin_copy_blocks, pin_copy_on_write_fork,
    pin_swap_round_trip,
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_block_rule_golden():
    """The allocation rule's block counts (golden fixture) for oracle and generator alike."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "blocks_rule.txt"))
            if l.strip() and not l.startswith("#")]
    for tokens, blocks in rows:
        assert oracle.blocks_for(int(tokens)) == int(blocks)
        assert workloads.blocks_needed(int(tokens)) == int(blocks)


@settings(max_examples=25, deadline=None)
@given(seed=st.integers(0, 10_000), dtype=st.sampled_from(["bf16", "f32"]),
       lengths=st.lists(st.integers(1, 70), min_size=1, max_size=4),
       kv=st.sampled_from([1, 2]), group=st.sampled_from([1, 2, 4]), D=st.sampled_from([4, 16, 64]))
def test_decode_brute_force_property(seed, dtype, lengths, kv, group, D):
    pin_decode_vs_sdpa(seed, tuple(lengths), Hq=kv * group, Hkv=kv, D=D, dtype=dtype)


@settings(max_examples=20, deadline=None)
@given(seed=st.integers(0, 10_000), cached=st.lists(st.integers(0, 40), min_size=1, max_size=3),
       new=st.integers(1, 33), group=st.sampled_from([1, 2, 4]))
def test_prefill_brute_force_property(seed, cached, new, group):
    pin_prefill_vs_sdpa(seed, tuple(cached), tuple([new] * len(cached)), Hq=2 * group, Hkv=2, D=8)


# ----------------------------------------------------------------------------- planted mistakes
MISTAKES = {
    "gqa head by modulo": ("kv_head_of", lambda h, g: h % 4),
    "causal aligned top-left": ("last_key", lambda row, n, L: row),
    "causal off by one": ("last_key", lambda row, n, L: L - n + row - 1),
    "blocks rounded down": ("blocks_for", lambda n: int(n) // 16),
    "bf16 decoded with wrong shift": (
        "to_float64",
        lambda bits, dt: ((bits.astype(np.uint32) << 15).view(np.float32).astype(np.float64)
                          if dt == "bf16" else np.asarray(bits, np.float32).astype(np.float64))),
    "scale 1/d": ("default_scale", lambda d: 1.0 / d),
    "slot as (offset, block)": ("slot_location", lambda s: (int(s) % 16, int(s) // 16)),
    "softmax over the wrong axis": (
        "softmax_weights",
        lambda s: np.nan_to_num(np.exp(s - s.max(0, keepdims=True))
                                / np.exp(s - s.max(0, keepdims=True)).sum(0, keepdims=True))),
    "values and keys swapped": (
        "attend",
        lambda q, k, v, lim, sc: pa_oracle.softmax_weights(
            np.where(np.arange(k.shape[0])[None, :] > np.asarray(lim)[:, None], -np.inf,
                     sc * (q @ v.T))) @ k),
    "block copy reversed": (
        "copy_blocks",
        lambda kp, vp, pairs: [kp.__setitem__(int(a), kp[int(b)]) or vp.__setitem__(int(a), vp[int(b)])
                               for a, b in np.asarray(pairs).reshape(-1, 2)] and None),
    "swap ignores its direction": (
        "swap_blocks",
        lambda kp, vp, hk, hv, pairs, to_host: [
            (hk.__setitem__(int(b), kp[int(a)]), hv.__setitem__(int(b), vp[int(a)]))
            for a, b in np.asarray(pairs).reshape(-1, 2)] and None),
    "table read backwards": (
        "gather_logical",
        lambda pool, row, L: pool[np.asarray(row[:(L + 15) // 16])[::-1]].reshape(
            (-1,) + pool.shape[2:])[:L]),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, wrong = MISTAKES[name]
    monkeypatch.setattr(pa_oracle, attr, wrong)
    failed = []
    for pin in ALL_PINS:
        try:
            pin()
        except Exception:  # noqa: BLE001 - any failure (assertion, index error) counts
            failed.append(pin.__name__)
    assert failed, f"no pin noticed the planted mistake {name!r}"
