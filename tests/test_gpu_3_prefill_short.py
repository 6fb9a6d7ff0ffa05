"""pa_prefill_chunk_short (chunks of a few rows through the decode kernel) on the GPU
against the fp64 oracle of causal chunked prefill.

Row i of a chunk of n rows sits at position seq_len - n + i and attends keys 0 ..
that position (arcyou teardown of vLLM paged attention, section "Continuous
batching: rebuild the batch every step"); the decode kernel's score tile then
holds (position, q head) columns, each with its own causal limit.
"""
import numpy as np
import pytest
import torch

import paged_kv_cache_245_amd as pa
import workloads
from gpu_support import as64, assert_close, device_tensor, gpu_pools, i32, run_prefill, run_prefill_short, say
from oracle_support import oracle_pools, oracle_prefill

pytestmark = pytest.mark.gpu


def check(w, what, **kw):
    d, k, v = gpu_pools(w)
    out = run_prefill_short(w, d, k, v, **kw)
    ok, ov = oracle_pools(w)
    assert_close(as64(out), oracle_prefill(w, ok, ov), "bf16", what)
    return d, k, v, out


@pytest.mark.parametrize("group,D", [(g, D) for g in (1, 2, 4, 8, 16) for D in (64, 128)])
def test_shapes(group, D):
    """Every group size at its largest chunk (16 / group rows), shorter chunks beside it, and
    chunks that start in one block and end in the next."""
    n = 16 // group
    cached = [0, 5, 16 - max(n // 2, 1), 100, 2000, 31]
    new = [1, n, n, max(n - 1, 1), n, 1]
    say(f"  short chunks G={group} D={D}, up to {n} rows")
    w = workloads.custom_prefill(500 + group + D, cached=cached, new=new, Hq=2 * group, Hkv=2, D=D, dtype="bf16")
    check(w, f"short G={group} D={D}")


def test_many_requests_records():
    """600 requests (more than the 256 workers), most of them read by one worker: their
    results wait in LDS records until the worker's range ends, and the records that do not
    fit are stored directly."""
    rng = np.random.default_rng(511)
    cached = rng.integers(0, 300, 600)
    new = rng.integers(1, 5, 600)
    say("  600 short chunks, G=4 D=128")
    w = workloads.custom_prefill(511, cached=cached.tolist(), new=new.tolist(), Hq=32, Hkv=8, D=128, dtype="bf16")
    check(w, "600 short chunks")


def test_most_requests():
    """8,192 requests, the most the call takes: the block prefix sums fill 32 KiB of the
    decode kernel's LDS beside its staged results; one more request is refused."""
    rng = np.random.default_rng(520)
    S = 8192
    cached = rng.integers(0, 120, S)
    new = rng.integers(1, 5, S)
    say("  8,192 short chunks, G=4 D=64")
    w = workloads.custom_prefill(520, cached=cached.tolist(), new=new.tolist(), Hq=8, Hkv=2, D=64, dtype="bf16")
    d, k, v, out = check(w, "8,192 short chunks")
    p = w.prefill
    assert pa.pa_prefill_chunk_short_workspace_size(d, S + 1, 4) == 0
    q = device_tensor(np.concatenate([p.q, p.q[:1]]), "bf16")
    with pytest.raises(pa.PAError) as e:
        pa.pa_prefill_chunk_short(d, torch.empty_like(q), q, k, v, i32(np.append(p.query_start_loc, q.shape[0])),
                                  i32(np.append(p.seq_lens, 1)), i32(np.concatenate([p.block_tables,
                                                                                     p.block_tables[:1]])),
                                  4, p.max_seq_len, w.scale, pa.chunk_short_workspace(d, S, 4))
    assert "num_seqs" in str(e.value)


def test_long_contexts_split():
    """Long contexts split over many workers: the merge combines partials per (request,
    position, head); a chunk's first keys and its own rows land in different workers."""
    say("  short chunks over long contexts")
    w = workloads.custom_prefill(512, cached=[30000, 8000, 12, 4095], new=[4, 3, 2, 4], Hq=32, Hkv=8, D=128,
                                 dtype="bf16")
    check(w, "long contexts")


def test_one_request_all_workers():
    """One request of 32,768 tokens whose last 4 are the chunk: every worker holds a piece."""
    say("  one 32,768-token request, 4-row chunk")
    w = workloads.custom_prefill(513, cached=[32764], new=[4], Hq=32, Hkv=8, D=128, dtype="bf16")
    check(w, "one long request")


@pytest.mark.parametrize("D", [64, 128])
def test_three_row_chunks(D):
    """Chunks of at most 3 rows over split contexts: the merge's wavefronts take 4 positions,
    the fourth of which no chunk has."""
    say(f"  three-row chunks D={D}")
    w = workloads.custom_prefill(519 + D, cached=[5000, 3000, 40, 7000], new=[3, 2, 3, 1], Hq=32, Hkv=8, D=D,
                                 dtype="bf16")
    check(w, f"three-row chunks D={D}")


def test_positions_beyond_chunks():
    """max_query_len above every chunk: positions no chunk has are skipped, in the kernel
    and in the merge."""
    say("  max_query_len 4 for chunks of at most 2 rows")
    w = workloads.custom_prefill(514, cached=[7, 3000, 40, 9000], new=[2, 1, 2, 2], Hq=16, Hkv=4, D=128,
                                 dtype="bf16")
    check(w, "positions beyond the chunks", max_query_len=4)


@pytest.mark.parametrize("seed", range(530, 538))
def test_random_sweep(seed):
    """Random group sizes, head dims, batch sizes, chunk lengths (up to the limit) and
    contexts (some ending inside a block, some a few thousand tokens long)."""
    rng = np.random.default_rng(seed)
    group = int(rng.choice([1, 2, 4, 8, 16]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    S = int(rng.integers(1, 40))
    n_max = 16 // group
    new = rng.integers(1, n_max + 1, S)
    cached = np.where(rng.random(S) < 0.3, rng.integers(0, 40, S), rng.integers(0, 3000, S))
    say(f"  random short chunks: seed {seed}, G={group}, Hkv={hkv}, D={D}, S={S}")
    w = workloads.custom_prefill(seed, cached=cached.tolist(), new=new.tolist(), Hq=group * hkv, Hkv=hkv, D=D,
                                 dtype="bf16")
    check(w, f"random sweep seed {seed}")


def test_empty_chunk_is_skipped():
    w = workloads.custom_prefill(515, cached=[3, 900], new=[2, 3], Hq=8, Hkv=2, D=64, dtype="bf16")
    d, k, v = gpu_pools(w)
    p = w.prefill
    q = device_tensor(p.q, "bf16")
    out = torch.zeros_like(q)
    # request 0's chunk is empty: rows 0..2 belong to request 1 (3 new rows of its 903)
    ws = pa.chunk_short_workspace(d, 2, 4)
    pa.pa_prefill_chunk_short(d, out, q[:3], k, v, i32([0, 0, 3]), i32([5, 903]), i32(p.block_tables), 4, 903,
                              w.scale, ws)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(as64(out[:3])))
    assert not out[3:].any()


def test_matches_prefill_chunk():
    """The same step through pa_prefill_chunk (MFMA query tiles) and through the short-chunk
    call agree to the bf16 output rounding."""
    rng = np.random.default_rng(516)
    cached = rng.integers(0, 4096, 64)
    new = rng.integers(1, 5, 64)
    w = workloads.custom_prefill(516, cached=cached.tolist(), new=new.tolist(), Hq=32, Hkv=8, D=128, dtype="bf16")
    d, k, v = gpu_pools(w)
    a = as64(run_prefill(w, d, k, v))
    b = as64(run_prefill_short(w, d, k, v))
    assert np.max(np.abs(a - b)) <= 2e-2


def test_bad_block_id():
    """An out-of-range block id inside a request's context makes that request's rows NaN and
    leaves the others as the oracle has them."""
    w = workloads.custom_prefill(517, cached=[100, 60], new=[3, 4], Hq=16, Hkv=4, D=128, dtype="bf16")
    d, k, v = gpu_pools(w)
    p = w.prefill
    tables = p.block_tables.copy()
    tables[1, 1] = w.spec.num_blocks + 5
    q = device_tensor(p.q, "bf16")
    out = torch.empty_like(q)
    ws = pa.chunk_short_workspace(d, 2, p.max_query_len)
    pa.pa_prefill_chunk_short(d, out, q, k, v, i32(p.query_start_loc), i32(p.seq_lens), i32(tables),
                              p.max_query_len, p.max_seq_len, w.scale, ws)
    torch.cuda.synchronize()
    o = as64(out)
    assert np.all(np.isnan(o[p.query_start_loc[1]:]))
    ok, ov = oracle_pools(w)
    ref = oracle_prefill(w, ok, ov)
    assert_close(o[:p.query_start_loc[1]], ref[:p.query_start_loc[1]], "bf16", "request beside a bad block")


def test_limits_and_workspace():
    w = workloads.custom_prefill(518, cached=[10], new=[2], Hq=16, Hkv=2, D=64, dtype="bf16")  # G = 8
    d, k, v = gpu_pools(w)
    p = w.prefill
    assert pa.pa_prefill_chunk_short_max_query_len(d) == 2
    assert pa.pa_prefill_chunk_short_workspace_size(d, 1, 3) == 0
    q = device_tensor(p.q, "bf16")
    out = torch.empty_like(q)
    args = (d, out, q, k, v, i32(p.query_start_loc), i32(p.seq_lens), i32(p.block_tables))
    with pytest.raises(pa.PAError) as e:
        pa.pa_prefill_chunk_short(*args, 3, p.max_seq_len, w.scale, pa.chunk_short_workspace(d, 1, 2))
    assert "max_query_len" in str(e.value)
    small = torch.empty(pa.pa_prefill_chunk_short_workspace_size(d, 1, 2) - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(pa.PAError) as e:
        pa.pa_prefill_chunk_short(*args, 2, p.max_seq_len, w.scale, small)
    assert "workspace" in str(e.value)
