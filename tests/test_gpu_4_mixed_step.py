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
