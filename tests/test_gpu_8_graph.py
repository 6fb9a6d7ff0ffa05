"""A whole continuous-batching step captured once in a HIP graph and replayed.

The step is pa_write_kv of the prefill rows, pa_prefill_chunk, and
pa_decode_append for the one-token requests; or, fused, pa_prefill_chunk_append
(which stores the prefill rows itself) and pa_decode_append. No call of the step allocates,
clears memory or synchronizes (outside PA_CHECK mode), so the step can be
captured. Each replay runs with new q/K/V copied into the captured buffers,
and its output and pools must equal, bit for bit, those of the same calls
launched one by one on a second pair of pools. That eager step runs between
the replays, with synchronizations in between.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_245_amd as pa
import workloads
from gpu_support import as64, assert_close, device_tensor, gpu_pools, i32, say
from oracle_support import oracle_decode, oracle_pools
from workloads import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("fused", [False, True])
def test_step_graph_replays_match_eager(fused):
    say(f"  graph capture of a mixed step (fused prefill: {fused})")
    w = workloads.custom_prefill(21, cached=[0, 40, 100], new=[30, 17, 64], Hq=8, Hkv=2, D=128,
                                 dtype="bf16", decode_lengths=[1, 16, 17, 200, 513])
    d, k0, v0 = gpu_pools(w, include_step=False)
    st, p, dec = w.step_write, w.prefill, w.decode
    P, T = w.num_prefills, p.q.shape[0]
    n_tok = st.key.shape[0]

    q = device_tensor(w.query, "bf16")
    key, value = device_tensor(st.key, "bf16"), device_tensor(st.value, "bf16")
    slots = i32(st.slot_mapping[:T])
    tables = i32(w.block_tables)
    qsl, seq = i32(p.query_start_loc), i32(p.seq_lens)
    lens = i32(dec.context_lens)
    ws = pa.decode_workspace(d, len(dec.context_lens), dec.max_context_len)
    scale = w.scale

    def step(k, v, out):
        if fused:
            pa.pa_prefill_chunk_append(d, out[:T], q[:T], key[:T], value[:T], k, v, qsl, seq, tables[:P],
                                       p.max_query_len, p.max_seq_len, scale)
        else:
            pa.pa_write_kv(d, key[:T], value[:T], k, v, slots)
            pa.pa_prefill_chunk(d, out[:T], q[:T], k, v, qsl, seq, tables[:P], p.max_query_len,
                                p.max_seq_len, scale)
        pa.pa_decode_append(d, out[T:], q[T:], key[T:], value[T:], k, v, tables[P:], lens,
                            dec.max_context_len, scale, ws)

    kg, vg = k0.clone(), v0.clone()
    out_g = torch.empty_like(q)
    ke, ve = k0.clone(), v0.clone()
    out_e = torch.empty_like(q)

    # one eager run on the side stream before capture, as torch asks
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(ke, ve, out_e)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(kg, vg, out_g)
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    outs = []
    for rep in range(3):
        # new inputs into the captured buffers, both pool pairs back to the set-up state
        q.copy_(torch.from_numpy(f32_to_bf16_bits(rng.standard_normal(tuple(q.shape), dtype=np.float32))
                                 .view(np.int16)).view(torch.bfloat16).cuda())
        for t in (key, value):
            t.copy_(torch.from_numpy(f32_to_bf16_bits(rng.standard_normal((n_tok,) + tuple(t.shape[1:]),
                                                                          dtype=np.float32))
                                     .view(np.int16)).view(torch.bfloat16).cuda())
        for dst, src in ((kg, k0), (vg, v0), (ke, k0), (ve, v0)):
            dst.copy_(src)
        out_g.zero_()
        out_e.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(ke, ve, out_e)  # eager work between the replays
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_g), bits(out_e)), f"replay {rep}: output"
        assert np.array_equal(bits(kg), bits(ke)) and np.array_equal(bits(vg), bits(ve)), f"replay {rep}: pools"
        assert np.all(np.isfinite(out_g.float().cpu().numpy()))
        outs.append(bits(out_g))
    assert not np.array_equal(outs[0], outs[1])  # the replays did see the new inputs


def test_decode_batch_steps_replayed_match_oracle():
    """The decode batch (64 requests, contexts 512-4096, 32/8 heads, D 128) as bench.py times
    it: several pa_decode_append calls captured in one HIP graph and replayed. Every replay
    leaves the pools as pa_write_kv of the newest tokens would, and the output matches the
    oracle and the eager call bit for bit."""
    say("  decode batch steps replayed from a graph")
    w = workloads.make(2)
    d, k, v = gpu_pools(w, include_step=False)
    dec, sw = w.decode, w.step_write
    S = len(dec.context_lens)
    q = device_tensor(dec.q, "bf16")
    key, value = device_tensor(sw.key, "bf16"), device_tensor(sw.value, "bf16")
    tables, lens = i32(dec.block_tables), i32(dec.context_lens)
    ws = pa.decode_workspace(d, S, dec.max_context_len)
    out_e, out_g = torch.empty_like(q), torch.empty_like(q)

    def call(out):
        pa.pa_decode_append(d, out, q, key, value, k, v, tables, lens, dec.max_context_len, w.scale, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_e)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = bits(out_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(4):
            call(out_g)
    ok, ov = oracle_pools(w)
    ref = oracle_decode(w, ok, ov)
    for rep in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_g), eager), f"replay {rep}: output differs from the eager call"
        call(out_e)  # eager work between the replays
        torch.cuda.synchronize()
    assert np.array_equal(k.view(torch.int16).cpu().numpy().view(np.uint16), ok)
    assert np.array_equal(v.view(torch.int16).cpu().numpy().view(np.uint16), ov)
    assert_close(as64(out_g), ref, "bf16", "decode batch, graph-replayed")


def test_shared_prefix_call_replayed_matches_eager():
    """pa_decode_shared_prefix (prefix pass, tails' decode, merge) captured in a HIP graph
    and replayed gives the eager call's output bit for bit, replay after replay."""
    say("  shared-prefix call replayed from a graph")
    w = workloads.c3_prefix_shared(seed=31, num_seqs=40)
    d, k, v = gpu_pools(w)
    dec = w.decode
    S = len(dec.context_lens)
    pb = w.shared_prefix_tokens // 16
    q = device_tensor(dec.q, "bf16")
    tables, lens = i32(dec.block_tables), i32(dec.context_lens)
    n = pa.pa_decode_shared_prefix_workspace_size(d, S, dec.max_context_len, pb)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    out_e, out_g = torch.empty_like(q), torch.empty_like(q)

    def call(out):
        pa.pa_decode_shared_prefix(d, out, q, k, v, tables, lens, dec.max_context_len, pb, w.scale, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_e)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = bits(out_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g)
    for rep in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_g), eager), f"replay {rep}"
        call(out_e)  # eager work between the replays
        torch.cuda.synchronize()
    ok, ov = oracle_pools(w)
    assert_close(as64(out_g), oracle_decode(w, ok, ov), "bf16", "shared prefix, graph-replayed")


def test_short_chunk_call_replayed_matches_eager():
    """pa_prefill_chunk_short (chunk kernel and merge; whole requests written through LDS
    records, split ones through the merge) captured in a HIP graph and replayed gives the
    eager call's output bit for bit, replay after replay, and the oracle's."""
    say("  short-chunk call replayed from a graph")
    rng = np.random.default_rng(32)
    cached = rng.integers(0, 3000, 48)
    w = workloads.custom_prefill(32, cached=cached.tolist(), new=rng.integers(1, 5, 48).tolist(), Hq=32, Hkv=8,
                                 D=128, dtype="bf16")
    d, k, v = gpu_pools(w)
    p = w.prefill
    q = device_tensor(p.q, "bf16")
    qsl, seq, tables = i32(p.query_start_loc), i32(p.seq_lens), i32(p.block_tables)
    ws = pa.chunk_short_workspace(d, 48, 4)
    out_e, out_g = torch.empty_like(q), torch.empty_like(q)

    def call(out):
        pa.pa_prefill_chunk_short(d, out, q, k, v, qsl, seq, tables, 4, p.max_seq_len, w.scale, ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(out_e)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = bits(out_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(out_g)
    for rep in range(3):
        out_g.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(bits(out_g), eager), f"replay {rep}"
        call(out_e)  # eager work between the replays
        torch.cuda.synchronize()
    ok, ov = oracle_pools(w)
    ref = oracle.prefill_chunk(p.q, ok, ov, p.query_start_loc, p.seq_lens, p.block_tables, "bf16", w.scale)
    assert_close(as64(out_g), ref, "bf16", "short chunks, graph-replayed")


def test_first_decode_call_inside_capture():
    """In a fresh process, the library's first decode call (pa_decode_append_noalloc) is made
    inside a graph capture, so its one-time set-up runs during the capture; replays must equal
    eager pa_decode_append bit for bit (tests/graph_first_call.py, run as a child process)."""
    import os
    import subprocess
    import sys
    say("  first decode call inside a graph capture (child process)")
    here = os.path.dirname(os.path.abspath(__file__))
    r = subprocess.run([sys.executable, "-u", os.path.join(here, "graph_first_call.py")], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0 and "first-call capture ok" in r.stdout, (r.stdout[-2000:], r.stderr[-2000:])
