"""CPU oracle for paged-KV attention (fp64, paged_attention) and plain models of the host
block pool (block_pool) and step scheduler (scheduler). TEST INFRASTRUCTURE: imported only by the tests, the smoke check and
the benchmark's CPU baseline; never by the HIP library, the host library or their bindings."""
from . import paged_attention  # noqa: F401
from .paged_attention import (  # noqa: F401
    BLOCK_SIZE,
    to_float64,
    empty_pool,
    slot_location,
    write_kv,
    copy_blocks,
    swap_blocks,
    blocks_for,
    gather_logical,
    kv_head_of,
    last_key,
    softmax_weights,
    attend,
    default_scale,
    decode,
    prefill_chunk,
    split_kv_decode,
    gather_kv,
)
