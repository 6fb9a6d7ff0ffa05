"""Copy-on-write block copies on the GPU: bit-exact against the oracle, and a forked request
that diverges after a copy (aitrending, "The 1960s Operating System Trick That Makes vLLM 4x
Faster", Technical Details)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_245_amd as pa
import workloads
from gpu_support import (as64, assert_close, desc_of, device_tensor, gpu_pools, host_bits, i32,
                         run_decode, say)
from oracle_support import oracle_pools

pytestmark = pytest.mark.gpu


def disjoint_pairs(num_blocks, n, seed):
    rng = np.random.default_rng(seed)
    perm = rng.permutation(num_blocks)
    dst = perm[:n]
    src = rng.choice(perm[n:], size=n, replace=True)  # sources may repeat
    return np.stack([src, dst], axis=1).astype(np.int32)


@pytest.mark.parametrize("index,n", [(1, 0), (1, 1), (1, 20), (2, 3000)])
def test_copy_blocks_bit_exact(index, n):
    say(f"  copy_blocks config {index}, {n} pairs")
    w = workloads.make(index)
    d, k, v = gpu_pools(w)
    ok, ov = oracle_pools(w)
    pairs = disjoint_pairs(w.spec.num_blocks, n, 5 + n)
    pa.pa_copy_blocks(d, k, v, i32(pairs.reshape(-1, 2)))
    torch.cuda.synchronize()
    oracle.copy_blocks(ok, ov, pairs)
    view = (lambda a: a.view(np.uint32)) if w.spec.dtype == "f32" else (lambda a: a)
    assert np.array_equal(view(host_bits(k)), view(ok))
    assert np.array_equal(view(host_bits(v)), view(ov))


def test_forked_request_diverges_after_copy():
    """Request B shares A's blocks; B's last block is copied before B writes its next token."""
    w = workloads.custom_decode(91, [37, 100], Hq=8, Hkv=2, D=128, dtype="bf16")
    d, k, v = gpu_pools(w)
    parent = host_bits(run_decode(w, d, k, v))
    dec = w.decode
    used = set(dec.block_tables[0, :3].tolist()) | set(dec.block_tables[1, :7].tolist())
    spare = next(b for b in range(w.spec.num_blocks) if b not in used)
    fork = dec.block_tables[:1].copy()
    pa.pa_copy_blocks(d, k, v, i32([[int(fork[0, 2]), spare]]))
    fork[0, 2] = spare
    rng = np.random.default_rng(7)
    new_k = workloads.f32_to_bf16_bits(rng.standard_normal((1, 2, 128), dtype=np.float32))
    new_v = workloads.f32_to_bf16_bits(rng.standard_normal((1, 2, 128), dtype=np.float32))
    pa.pa_write_kv(d, device_tensor(new_k, "bf16"), device_tensor(new_v, "bf16"), k, v,
                   i32([spare * 16 + 5]))
    again = host_bits(run_decode(w, d, k, v))
    assert np.array_equal(again, parent), "the parent must not see the fork's write"
    # the fork's query: request A's query, context = A's 37 tokens + the new one
    q = device_tensor(dec.q[:1], "bf16")
    out = torch.empty_like(q)
    pa.pa_decode(d, out, q, k, v, i32(fork), i32([38]), 38, w.scale, pa.decode_workspace(d, 1, 38))
    torch.cuda.synchronize()
    ok, ov = oracle_pools(w)
    oracle.copy_blocks(ok, ov, [[int(dec.block_tables[0, 2]), spare]])
    oracle.write_kv(ok, ov, new_k, new_v, np.array([spare * 16 + 5], np.int32))
    ref = oracle.decode(dec.q[:1], ok, ov, fork, np.array([38], np.int32), "bf16", w.scale)
    assert_close(as64(out), ref, "bf16", "forked request")


def test_copy_blocks_checks(monkeypatch):
    w = workloads.custom_decode(93, [40], Hq=4, Hkv=2, D=64, dtype="bf16")
    d, k, v = gpu_pools(w)
    before = host_bits(k).copy()
    pa.pa_copy_blocks(d, k, v, i32([[0, w.spec.num_blocks + 2], [-1, 1]]))  # skipped
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(k), before)
    monkeypatch.setenv("PA_CHECK", "1")
    for bad in ([[0, 1], [2, 1]], [[0, 1], [1, 2]], [[0, w.spec.num_blocks]]):
        with pytest.raises(pa.PAError) as e:
            pa.pa_copy_blocks(d, k, v, i32(bad))
        assert e.value.status == -4


def pinned_host_pool(w, num_host_blocks, fill=0):
    s = w.spec
    shape = (num_host_blocks, 16, s.num_kv_heads, s.head_dim)
    dt = torch.bfloat16 if s.dtype == "bf16" else torch.float32
    t = torch.empty(shape, dtype=dt, pin_memory=True)
    t.view(torch.int16 if s.dtype == "bf16" else torch.int32).fill_(fill)
    return t


def host_pool_bits(t):
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


@pytest.mark.parametrize("index,n", [(1, 1), (1, 13), (2, 2000)])
def test_swap_out_and_in_bit_exact(index, n):
    """Swap n blocks out to a pinned host pool and back into other device blocks: both
    directions bit-exact against the oracle, every other block untouched."""
    say(f"  swap config {index}, {n} blocks")
    w = workloads.make(index)
    d, k, v = gpu_pools(w)
    ok, ov = oracle_pools(w)
    nh = n + 7
    hk, hv = pinned_host_pool(w, nh), pinned_host_pool(w, nh)
    ohk, ohv = host_pool_bits(hk).copy(), host_pool_bits(hv).copy()
    rng = np.random.default_rng(n)
    perm = rng.permutation(w.spec.num_blocks)
    src, dst = perm[:n], perm[n:2 * n] if 2 * n <= w.spec.num_blocks else perm[:n][::-1].copy()
    hosts = rng.permutation(nh)[:n]
    out_pairs = np.stack([src, hosts], 1).astype(np.int32)
    view = (lambda a: a.view(np.uint32)) if w.spec.dtype == "f32" else (lambda a: a)
    pa.pa_swap_blocks(d, k, v, hk, hv, i32(out_pairs), pa.PA_SWAP_OUT)
    torch.cuda.synchronize()
    oracle.swap_blocks(ok, ov, ohk, ohv, out_pairs, True)
    assert np.array_equal(view(host_pool_bits(hk)), view(ohk))
    assert np.array_equal(view(host_pool_bits(hv)), view(ohv))
    in_pairs = np.stack([hosts, dst], 1).astype(np.int32)
    pa.pa_swap_blocks(d, k, v, hk, hv, i32(in_pairs), pa.PA_SWAP_IN)
    torch.cuda.synchronize()
    oracle.swap_blocks(ok, ov, ohk, ohv, in_pairs, False)
    assert np.array_equal(view(host_bits(k)), view(ok))
    assert np.array_equal(view(host_bits(v)), view(ov))


def test_swapped_request_decodes_identically():
    """A request whose blocks went to the host and came back into other blocks gives a
    bit-identical decode through its new table."""
    w = workloads.custom_decode(93, [300, 45], Hq=8, Hkv=2, D=128, dtype="bf16", num_blocks=64)
    d, k, v = gpu_pools(w)
    before = host_bits(run_decode(w, d, k, v))
    dec = w.decode
    nb = (int(dec.context_lens[0]) + 15) // 16
    table = dec.block_tables[0, :nb].copy()
    used = set(dec.block_tables.ravel().tolist())
    fresh = np.array([b for b in range(w.spec.num_blocks) if b not in used][:nb], np.int32)
    hk, hv = pinned_host_pool(w, nb), pinned_host_pool(w, nb)
    pa.pa_swap_blocks(d, k, v, hk, hv, i32(np.stack([table, np.arange(nb)], 1)), pa.PA_SWAP_OUT)
    k[torch.from_numpy(table.astype(np.int64)).cuda()] = 0  # the old blocks get reused
    pa.pa_swap_blocks(d, k, v, hk, hv, i32(np.stack([np.arange(nb), fresh], 1)), pa.PA_SWAP_IN)
    tables = dec.block_tables.copy()
    tables[0, :nb] = fresh
    after = host_bits(run_decode(w, d, k, v, tables=tables))
    assert np.array_equal(after, before)


def test_swap_refuses_pageable_host_memory():
    w = workloads.make(1)
    d, k, v = gpu_pools(w)
    lib = pa.load()
    import ctypes
    pageable = np.zeros(4 * 16 * w.spec.num_kv_heads * w.spec.head_dim, np.float32)
    p = ctypes.c_void_p(pageable.ctypes.data)
    pairs = i32(np.array([[0, 0]]))
    st = lib.pa_swap_blocks(ctypes.byref(d), ctypes.c_void_p(k.data_ptr()), ctypes.c_void_p(v.data_ptr()),
                            p, p, 4, ctypes.c_void_p(pairs.data_ptr()), 1, pa.PA_SWAP_OUT, None)
    assert st == -1


def test_swap_checks(monkeypatch):
    w = workloads.make(1)
    d, k, v = gpu_pools(w)
    hk, hv = pinned_host_pool(w, 4), pinned_host_pool(w, 4)
    monkeypatch.setenv("PA_CHECK", "1")
    for bad in ([[0, 4]], [[w.spec.num_blocks, 0]], [[0, 1], [2, 1]]):
        with pytest.raises(pa.PAError):
            pa.pa_swap_blocks(d, k, v, hk, hv, i32(np.array(bad)), pa.PA_SWAP_OUT)
