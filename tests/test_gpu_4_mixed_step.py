"""One continuous-batching step on one stream: write the new tokens' K/V, run the chunked
prefills, then the decodes (arcyou teardown of vLLM, section "Continuous batching")."""
import numpy as np
import pytest
import torch

import paged_kv_cache_245_amd as pa
import workloads
from gpu_support import (as64, assert_close, device_tensor, gpu_pools, host_bits, i32, say)
from oracle_support import oracle_decode, oracle_pools, oracle_prefill

pytestmark = pytest.mark.gpu


def test_mixed_step():
    say("  mixed step config 4")
    w = workloads.make(4)
    d, k, v = gpu_pools(w, include_step=False)
    st, p, dec = w.step_write, w.prefill, w.decode
    q_all = device_tensor(w.query, "bf16")
    out = torch.empty_like(q_all)
    T = p.q.shape[0]
    ws = pa.decode_workspace(d, len(dec.context_lens), dec.max_context_len)
    tables = i32(w.block_tables)
    pa.pa_write_kv(d, device_tensor(st.key, "bf16"), device_tensor(st.value, "bf16"), k, v,
                   i32(st.slot_mapping))
    pa.pa_prefill_chunk(d, out[:T], q_all[:T], k, v, i32(p.query_start_loc), i32(p.seq_lens),
                        tables[:w.num_prefills], p.max_query_len, p.max_seq_len, w.scale)
    pa.pa_decode(d, out[T:], q_all[T:], k, v, tables[w.num_prefills:], i32(dec.context_lens),
                 dec.max_context_len, w.scale, ws)
    torch.cuda.synchronize()
    ok, ov = oracle_pools(w)
    assert np.array_equal(host_bits(k), ok) and np.array_equal(host_bits(v), ov)
    got = as64(out)
    assert_close(got[:T], oracle_prefill(w, ok, ov), "bf16", "step prefill")
    assert_close(got[T:], oracle_decode(w, ok, ov), "bf16", "step decode")


def test_mixed_step_two_streams():
    """The step as the step runner issues it: the prefill rows written, then the chunked
    prefill on the caller's stream and pa_decode_append_lean (storing the decode tokens) on
    a second stream forked after the write and joined at the end. Pools and prefill rows
    equal those of the one-stream step (pa_decode_append) bit for bit; both steps' decode
    outputs match the oracle."""
    say("  mixed step config 4, decode on a second stream")
    w = workloads.make(4)
    st, p, dec = w.step_write, w.prefill, w.decode
    q_all = device_tensor(w.query, "bf16")
    T = p.q.shape[0]
    key, value = device_tensor(st.key, "bf16"), device_tensor(st.value, "bf16")
    slots = i32(st.slot_mapping)
    tables = i32(w.block_tables)
    qsl, seq, lens = i32(p.query_start_loc), i32(p.seq_lens), i32(dec.context_lens)
    P = w.num_prefills

    def step(k, v, out, ws, side):
        main = torch.cuda.current_stream()
        pa.pa_write_kv(d, key[:T], value[:T], k, v, slots[:T])
        if side is not None:
            side.wait_stream(main)
        pa.pa_prefill_chunk(d, out[:T], q_all[:T], k, v, qsl, seq, tables[:P], p.max_query_len,
                            p.max_seq_len, w.scale)
        call = pa.pa_decode_append if side is None else pa.pa_decode_append_lean
        call(d, out[T:], q_all[T:], key[T:], value[T:], k, v, tables[P:], lens, dec.max_context_len,
             w.scale, ws, stream=side)
        if side is not None:
            main.wait_stream(side)

    d, k1, v1 = gpu_pools(w, include_step=False)
    k2, v2 = k1.clone(), v1.clone()
    out1, out2 = torch.empty_like(q_all), torch.empty_like(q_all)
    ws1 = pa.decode_workspace(d, len(dec.context_lens), dec.max_context_len)
    ws2 = pa.decode_workspace(d, len(dec.context_lens), dec.max_context_len)
    step(k1, v1, out1, ws1, None)
    step(k2, v2, out2, ws2, torch.cuda.Stream())
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out1)[:T], host_bits(out2)[:T])
    assert np.array_equal(host_bits(k1), host_bits(k2)) and np.array_equal(host_bits(v1), host_bits(v2))
    ok, ov = oracle_pools(w)
    assert np.array_equal(host_bits(k2), ok) and np.array_equal(host_bits(v2), ov)
    got = as64(out2)
    assert_close(got[:T], oracle_prefill(w, ok, ov), "bf16", "two-stream step prefill")
    ref = oracle_decode(w, ok, ov)
    assert_close(got[T:], ref, "bf16", "two-stream step decode (lean)")
    assert_close(as64(out1)[T:], ref, "bf16", "one-stream step decode")


def test_mixed_step_fused_two_streams():
    """The step with no separate write: pa_prefill_chunk_append (which stores the prefill rows)
    on the caller's stream and pa_decode_append_lean (which stores the decode tokens) on a
    second stream, both forked at the start of the step. Pools and prefill rows equal those of
    the one-stream step (write, prefill, pa_decode_append) bit for bit; the decode matches the
    oracle."""
    say("  mixed step config 4, fused prefill and decode on two streams")
    w = workloads.make(4)
    st, p, dec = w.step_write, w.prefill, w.decode
    q_all = device_tensor(w.query, "bf16")
    T = p.q.shape[0]
    key, value = device_tensor(st.key, "bf16"), device_tensor(st.value, "bf16")
    slots = i32(st.slot_mapping)
    tables = i32(w.block_tables)
    qsl, seq, lens = i32(p.query_start_loc), i32(p.seq_lens), i32(dec.context_lens)
    P = w.num_prefills
    d, k1, v1 = gpu_pools(w, include_step=False)
    k2, v2 = k1.clone(), v1.clone()
    out1, out2 = torch.empty_like(q_all), torch.empty_like(q_all)
    ws1 = pa.decode_workspace(d, len(dec.context_lens), dec.max_context_len)
    ws2 = pa.decode_workspace(d, len(dec.context_lens), dec.max_context_len)
    # one stream, separate write
    pa.pa_write_kv(d, key[:T], value[:T], k1, v1, slots[:T])
    pa.pa_prefill_chunk(d, out1[:T], q_all[:T], k1, v1, qsl, seq, tables[:P], p.max_query_len,
                        p.max_seq_len, w.scale)
    pa.pa_decode_append(d, out1[T:], q_all[T:], key[T:], value[T:], k1, v1, tables[P:], lens,
                        dec.max_context_len, w.scale, ws1)
    # two streams, no write
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    side.wait_stream(main)
    pa.pa_prefill_chunk_append(d, out2[:T], q_all[:T], key[:T], value[:T], k2, v2, qsl, seq, tables[:P],
                               p.max_query_len, p.max_seq_len, w.scale)
    pa.pa_decode_append_lean(d, out2[T:], q_all[T:], key[T:], value[T:], k2, v2, tables[P:], lens,
                             dec.max_context_len, w.scale, ws2, stream=side)
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out1)[:T], host_bits(out2)[:T])
    assert np.array_equal(host_bits(k1), host_bits(k2)) and np.array_equal(host_bits(v1), host_bits(v2))
    ok, ov = oracle_pools(w)
    assert np.array_equal(host_bits(k2), ok) and np.array_equal(host_bits(v2), ov)
    got = as64(out2)
    assert_close(got[:T], oracle_prefill(w, ok, ov), "bf16", "fused two-stream step prefill")
    assert_close(got[T:], oracle_decode(w, ok, ov), "bf16", "fused two-stream step decode (lean)")
