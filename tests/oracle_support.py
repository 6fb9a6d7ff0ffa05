"""Test helpers that drive the fp64 oracle from a seeded workload."""
import numpy as np

import oracle
from workloads import POISON_BITS


def oracle_pools(w, include_step=True):
    """Oracle pools after set-up writes (and the step's writes), starting from NaN poison."""
    s = w.spec
    k = oracle.empty_pool(s.num_blocks, s.num_kv_heads, s.head_dim, s.dtype, POISON_BITS[s.dtype])
    v = oracle.empty_pool(s.num_blocks, s.num_kv_heads, s.head_dim, s.dtype, POISON_BITS[s.dtype])
    su = w.setup
    oracle.write_kv(k, v, su.key, su.value, su.slot_mapping)
    if include_step:
        st = w.step_write
        oracle.write_kv(k, v, st.key, st.value, st.slot_mapping)
    return k, v


def oracle_decode(w, k, v, pairs=None):
    d = w.decode
    return oracle.decode(d.q, k, v, d.block_tables, d.context_lens, w.spec.dtype, w.scale, pairs=pairs)


def oracle_prefill(w, k, v):
    p = w.prefill
    return oracle.prefill_chunk(p.q, k, v, p.query_start_loc, p.seq_lens, p.block_tables,
                                w.spec.dtype, w.scale)


def values64(bits, dtype):
    """float64 of storage bits through torch's own bfloat16/float32 conversion (not the oracle's)."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
        return t.to(torch.float64).numpy()
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(torch.float64).numpy()
