"""MI355X-native attention over a paged KV cache: Python face of libpa.so.

The calls mirror include/pa.h one to one (pa_write_kv, pa_decode,
pa_prefill_chunk, ...) and take torch tensors; all compute runs in the gfx950
HIP kernels of libpa.so.
"""
from ._lib import (  # noqa: F401
    BLOCK_SIZE,
    EXPORTED,
    PA_BF16,
    PA_F32,
    PA_SWAP_IN,
    PA_SWAP_OUT,
    CacheDesc,
    PAError,
    cache_desc,
    decode_workspace,
    load,
    pa_bench_copy,
    pa_bench_flush,
    pa_bench_read,
    pa_copy_blocks,
    pa_decode,
    pa_decode_append,
    pa_decode_append_lean,
    pa_decode_partition_tokens,
    pa_decode_shared_prefix,
    pa_decode_shared_prefix_workspace_size,
    pa_decode_workspace_size,
    pa_gather_kv,
    pa_last_error_detail,
    pa_prefill_chunk,
    pa_strerror,
    pa_swap_blocks,
    pa_version,
    pa_write_kv,
    torch_dtype,
)
