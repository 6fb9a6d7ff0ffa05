"""Slot writes and block-table gathers on the GPU: bit-exact against the oracle, over every
slot of the pool (untouched and NaN-poisoned slots included)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_245_amd as pa
import workloads
from gpu_support import desc_of, gpu_pools, host_bits, i32, device_tensor, poisoned_pool, say
from oracle_support import oracle_pools

pytestmark = pytest.mark.gpu


def as_uint(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_pool_equal(gpu, ref, what):
    g, r = as_uint(host_bits(gpu)), as_uint(ref)
    bad = np.argwhere(g != r)
    assert len(bad) == 0, f"{what}: {len(bad)} elements differ, first at {bad[0].tolist()}"


@pytest.mark.parametrize("index", [1, 4])
def test_write_bit_exact(index):
    say(f"  write_kv config {index}")
    w = workloads.make(index)
    d, k, v = gpu_pools(w)
    torch.cuda.synchronize()
    ok, ov = oracle_pools(w)
    assert_pool_equal(k, ok, "k pool")
    assert_pool_equal(v, ov, "v pool")


def test_skip_slots_and_ragged_counts():
    w = workloads.custom_decode(41, [3, 17, 33, 1, 64], Hq=8, Hkv=4, D=64, dtype="bf16")
    su = w.setup
    slots = su.slot_mapping.copy()
    slots[::3] = -1  # these tokens must not be written
    d = desc_of(w)
    for n in (0, 1, 7, len(slots)):  # empty, single, ragged, all
        k, v = poisoned_pool(w), poisoned_pool(w)
        pa.pa_write_kv(d, device_tensor(su.key[:n], "bf16"), device_tensor(su.value[:n], "bf16"),
                       k, v, i32(slots[:n]))
        torch.cuda.synchronize()
        s = w.spec
        ok = oracle.empty_pool(s.num_blocks, s.num_kv_heads, s.head_dim, "bf16", 0x7FC0)
        ov = ok.copy()
        oracle.write_kv(ok, ov, su.key[:n], su.value[:n], slots[:n])
        assert_pool_equal(k, ok, f"k pool, {n} tokens")
        assert_pool_equal(v, ov, f"v pool, {n} tokens")


@pytest.mark.parametrize("index", [1, 2])
def test_gather_bit_exact(index):
    say(f"  gather_kv config {index}")
    w = workloads.make(index)
    d, k, v = gpu_pools(w)
    dec = w.decode
    S, L = len(dec.context_lens), dec.max_context_len
    s = w.spec
    dk = torch.zeros((S, L, s.num_kv_heads, s.head_dim), dtype=k.dtype, device="cuda")
    dv = torch.zeros_like(dk)
    pa.pa_gather_kv(d, dk, dv, k, v, i32(dec.block_tables), i32(dec.context_lens), L)
    torch.cuda.synchronize()
    gk, gv = as_uint(host_bits(dk)), as_uint(host_bits(dv))
    ok, ov = oracle_pools(w)
    rk = oracle.gather_kv(ok, dec.block_tables, dec.context_lens)
    rv = oracle.gather_kv(ov, dec.block_tables, dec.context_lens)
    for r in range(S):
        n = int(dec.context_lens[r])
        assert np.array_equal(gk[r, :n], as_uint(rk[r])), r
        assert np.array_equal(gv[r, :n], as_uint(rv[r])), r
        assert not gk[r, n:].any()  # rows past the context are left untouched (zeros)
