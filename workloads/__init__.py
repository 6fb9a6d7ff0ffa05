"""Seeded synthetic inputs for paged-KV attention (lengths, placement, tables, Q/K/V).

Shared by the oracle-side tests and the HIP-side tests and benchmark; holds no
attention arithmetic.
"""
from .configs import (  # noqa: F401
    BLOCK_SIZE,
    POISON_BITS,
    PoolSpec,
    KVWrite,
    DecodeBatch,
    PrefillBatch,
    Workload,
    f32_to_bf16_bits,
    blocks_needed,
    c1_tiny_decode,
    c2_decode_batch,
    c3_prefix_shared,
    c4_mixed_step,
    c5_long_decode,
    custom_decode,
    custom_prefill,
    make,
    CONFIG_NAMES,
)
