"""Structure of the seeded workloads (CPU only): block counts, placement, slots, sharing."""
import numpy as np
import pytest

import workloads
from workloads import blocks_needed


def check_structure(w):
    s = w.spec
    R = w.num_requests
    assert w.block_tables.shape[0] == R
    assert len(w.slots) == len(w.key_tokens) == len(w.value_tokens)
    # slots are distinct and inside the pool
    assert len(np.unique(w.slots)) == len(w.slots)
    assert w.slots.min() >= 0 and w.slots.max() < s.num_blocks * 16
    prefix_blocks = w.shared_prefix_tokens // 16
    owned = []
    for r in range(R):
        nb = blocks_needed(w.lengths[r])
        row = w.block_tables[r]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < s.num_blocks)
        owned.append(row[prefix_blocks:nb])
        # every logical position's slot is the table's block * 16 + offset
        pos = np.arange(w.lengths[r])
        want = row[pos // 16].astype(np.int64) * 16 + pos % 16
        assert np.array_equal(w.slots[w.token_index[r]], want)
    owned = np.concatenate(owned)
    assert len(np.unique(owned)) == len(owned), "private blocks are not shared"
    # the step writes exactly each request's new tokens, prefills then decodes
    n_step = len(w.slots) - w.num_setup_tokens
    assert n_step == int(w.new_tokens.sum())
    assert w.query.shape == (int(w.new_tokens[:w.num_prefills].sum()) + R - w.num_prefills,
                             s.num_q_heads, s.head_dim)


def test_c1():
    w = workloads.make(1)
    check_structure(w)
    assert w.lengths.tolist() == [1, 17, 48, 100]
    assert w.spec.num_blocks == 64 and w.spec.dtype == "f32"
    used = {int(b) for r in range(4) for b in w.block_tables[r, :blocks_needed(w.lengths[r])]}
    assert len(used) == 13
    assert w.scale == 1 / 8


def test_c2_full_size():
    w = workloads.make(2)
    check_structure(w)
    need = sum(blocks_needed(L) for L in w.lengths)
    assert w.spec.num_blocks == -(-need * 11 // 10)
    assert w.lengths.min() >= 512 and w.lengths.max() <= 4096
    assert w.key_tokens.dtype == np.uint16


def test_c3_shape_small():
    w = workloads.c3_prefix_shared(seed=3, num_seqs=12, prefix_tokens=64, tail_lo=5, tail_hi=40,
                                   Hq=4, Hkv=2, D=16)
    check_structure(w)
    assert np.all(w.block_tables[:, :4] == w.block_tables[0, :4])


def test_c4_shape_small():
    w = workloads.c4_mixed_step(seed=4, num_prefills=3, new_tokens=40, cached_hi=50,
                                num_decodes=5, dec_lo=3, dec_hi=70, Hq=4, Hkv=2, D=16)
    check_structure(w)
    p, d = w.prefill, w.decode
    assert p.query_start_loc.tolist() == [0, 40, 80, 120]
    assert d.q.shape[0] == 5


def test_c5_shape_small():
    w = workloads.c5_long_decode(seed=5, num_seqs=2, length=512, Hq=8, Hkv=2, D=16)
    check_structure(w)
    assert w.spec.num_blocks == 64
    assert sorted(w.block_tables.ravel().tolist()) == list(range(64))


def test_seeded_and_repeatable():
    a = workloads.make(1)
    b = workloads.make(1)
    assert np.array_equal(a.key_tokens, b.key_tokens) and np.array_equal(a.block_tables, b.block_tables)
    c = workloads.make(1, seed=101)
    assert not np.array_equal(a.key_tokens, c.key_tokens)


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    assert bits.tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]
