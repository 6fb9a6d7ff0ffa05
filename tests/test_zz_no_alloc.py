"""pa_decode_append_noalloc (the decode-append call whose split-KV partials live in the
library's fixed per-GPU scratch array instead of a caller's workspace) against
pa_decode_append through the C ABI: two calls in a row, the second smaller, each
output and the pools bit-identical to the workspace call's; sizes beyond the
array are refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest
import torch

import paged_kv_cache_245_amd as pa
import workloads
from gpu_support import as64, assert_close, device_tensor, gpu_pools, host_bits, i32, say
from oracle_support import oracle_decode, oracle_pools

pytestmark = pytest.mark.gpu


def run_both(w):
    """The step's decode through pa_decode_append (with a workspace) and through
    pa_decode_append_noalloc, each on its own copy of the pools (the step not yet written)."""
    dec, sw = w.decode, w.step_write
    S = len(dec.context_lens)
    dt = w.spec.dtype
    q = device_tensor(dec.q, dt)
    key, value = device_tensor(sw.key, dt), device_tensor(sw.value, dt)
    tables, lens = i32(dec.block_tables), i32(dec.context_lens)
    results = []
    for noalloc in (False, True):
        d, k, v = gpu_pools(w, include_step=False)
        out = torch.full_like(q, float("nan"))
        if noalloc:
            pa.pa_decode_append_noalloc(d, out, q, key, value, k, v, tables, lens, dec.max_context_len, w.scale)
        else:
            ws = pa.decode_workspace(d, S, dec.max_context_len, 0)
            pa.pa_decode_append(d, out, q, key, value, k, v, tables, lens, dec.max_context_len, w.scale, ws)
        torch.cuda.synchronize()
        results.append((host_bits(out), host_bits(k), host_bits(v), as64(out)))
    return results


def test_noalloc_matches_workspace_call_twice():
    """Two calls in a row, the second with a smaller input: the scratch array keeps the first
    call's contents, which must not leak into the second."""
    cases = [("64 requests, 512..4096 tokens", workloads.c2_decode_batch(seed=21)),
             ("8 requests, 1..600 tokens", workloads.custom_decode(22, np.random.default_rng(22).integers(1, 601, 8).tolist(),
                                                                 Hq=32, Hkv=8, D=128, dtype="bf16"))]
    for what, w in cases:
        say(f"  noalloc vs workspace call: {what}")
        (o1, k1, v1, f1), (o2, k2, v2, f2) = run_both(w)
        assert np.array_equal(o1, o2), f"{what}: outputs differ"
        assert np.array_equal(k1, k2) and np.array_equal(v1, v2), f"{what}: pools differ"
        ok, ov = oracle_pools(w)
        assert np.array_equal(k2, ok) and np.array_equal(v2, ov), f"{what}: pools differ from the oracle's"
        assert_close(f2, oracle_decode(w, ok, ov), "bf16", f"noalloc, {what}")


def test_noalloc_fixed_partitions_and_long_requests():
    """Fixed partitions (partition_tokens 64) and a few requests split over every worker (the
    wide merge), each against the workspace call."""
    w = workloads.custom_decode(23, [5000, 3, 17000, 800], Hq=16, Hkv=2, D=128, dtype="bf16")
    dec, sw = w.decode, w.step_write
    q = device_tensor(dec.q, "bf16")
    key, value = device_tensor(sw.key, "bf16"), device_tensor(sw.value, "bf16")
    tables, lens = i32(dec.block_tables), i32(dec.context_lens)
    for part in (0, 64):
        outs = []
        for noalloc in (False, True):
            d, k, v = gpu_pools(w, include_step=False)
            out = torch.empty_like(q)
            if noalloc:
                pa.pa_decode_append_noalloc(d, out, q, key, value, k, v, tables, lens, dec.max_context_len,
                                            w.scale, partition_tokens=part)
            else:
                pa.pa_decode_append(d, out, q, key, value, k, v, tables, lens, dec.max_context_len, w.scale,
                                    pa.decode_workspace(d, 4, dec.max_context_len, part), part)
            torch.cuda.synchronize()
            outs.append((host_bits(out), host_bits(k), host_bits(v)))
        assert all(np.array_equal(a, b) for a, b in zip(*outs)), f"partition {part}: results differ"


def test_noalloc_refuses_oversized_batches():
    """A batch whose workspace exceeds the fixed array is refused before any launch, with the
    sizes named."""
    lib = pa.load()
    d = pa.cache_desc(32, 8, 128, 1 << 20, "bf16")
    S = 4096
    assert pa.pa_decode_workspace_size(d, S, 8192) > pa.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the size check fails first
    st = lib.pa_decode_append_noalloc(ctypes.byref(d), fake, fake, fake, fake, fake, fake, fake, 512, fake,
                                      S, 8192, 0.088, 0, None)
    assert st == -3
    assert "fixed" in pa.pa_last_error_detail()
