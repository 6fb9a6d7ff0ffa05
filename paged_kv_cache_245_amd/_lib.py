"""ctypes binding of libpa.so: the C calls of include/pa.h, taking torch tensors.

Argument marshalling only: shapes and dtypes are checked, device pointers and
the current HIP stream are passed through, and a non-zero status raises
PAError. Every step of attention runs in the library's HIP kernels; there is
no fallback. torch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpa.so")
_lib = None

PA_F32 = 0
PA_BF16 = 1
BLOCK_SIZE = 16

EXPORTED = ("pa_write_kv", "pa_decode_partition_tokens", "pa_decode_workspace_size", "pa_decode",
            "pa_decode_append", "pa_decode_append_lean", "pa_decode_append_noalloc",
            "pa_decode_shared_prefix_workspace_size", "pa_decode_shared_prefix",
            "pa_prefill_chunk", "pa_prefill_chunk_append", "pa_prefill_chunk_short_max_query_len",
            "pa_prefill_chunk_short_workspace_size", "pa_prefill_chunk_short", "pa_copy_blocks", "pa_swap_blocks", "pa_gather_kv", "pa_strerror", "pa_last_error_detail",
            "pa_version", "pa_bench_copy", "pa_bench_read", "pa_bench_flush", "pa_bench_mfma")


class PAError(RuntimeError):
    def __init__(self, status: int, call: str):
        lib = load()
        msg = lib.pa_strerror(status).decode()
        detail = lib.pa_last_error_detail().decode()
        super().__init__(f"{call}: {msg} ({status}){': ' + detail if detail else ''}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_blocks", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


def cache_desc(num_q_heads, num_kv_heads, head_dim, num_blocks, dtype) -> CacheDesc:
    """dtype: "bf16"/"f32" or torch.bfloat16/torch.float32."""
    code = {"bf16": PA_BF16, "f32": PA_F32, torch.bfloat16: PA_BF16, torch.float32: PA_F32}[dtype]
    return CacheDesc(num_q_heads, num_kv_heads, head_dim, BLOCK_SIZE, num_blocks, code, 0)


def torch_dtype(desc: CacheDesc):
    return torch.bfloat16 if desc.dtype == PA_BF16 else torch.float32


def load():
    """Load libpa.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                           "`python -m paged_kv_cache_245_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I32, I64, SZ, F = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    D = ctypes.POINTER(CacheDesc)
    sig = {
        "pa_write_kv": (ctypes.c_int, [D, P, P, P, P, P, I64, P]),
        "pa_decode_partition_tokens": (I32, [D, I32, I32]),
        "pa_decode_workspace_size": (SZ, [D, I32, I32, I32]),
        "pa_decode": (ctypes.c_int, [D, P, P, P, P, P, I32, P, I32, I32, F, I32, P, SZ, P]),
        "pa_decode_append": (ctypes.c_int, [D, P, P, P, P, P, P, P, I32, P, I32, I32, F, I32, P, SZ, P]),
        "pa_decode_append_lean": (ctypes.c_int, [D, P, P, P, P, P, P, P, I32, P, I32, I32, F, P, SZ, P]),
        "pa_decode_append_noalloc": (ctypes.c_int, [D, P, P, P, P, P, P, P, I32, P, I32, I32, F, I32, P]),
        "pa_decode_shared_prefix_workspace_size": (SZ, [D, I32, I32, I32]),
        "pa_decode_shared_prefix": (ctypes.c_int, [D, P, P, P, P, P, I32, P, I32, I32, I32, F, P, SZ, P]),
        "pa_prefill_chunk": (ctypes.c_int, [D, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F, P]),
        "pa_prefill_chunk_append": (ctypes.c_int, [D, P, P, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F, P]),
        "pa_prefill_chunk_short_max_query_len": (I32, [D]),
        "pa_prefill_chunk_short_workspace_size": (SZ, [D, I32, I32]),
        "pa_prefill_chunk_short": (ctypes.c_int, [D, P, P, P, P, P, P, P, I32, I32, I32, I32, I32, F, P, SZ, P]),
        "pa_copy_blocks": (ctypes.c_int, [D, P, P, P, I64, P]),
        "pa_swap_blocks": (ctypes.c_int, [D, P, P, P, P, I64, P, I64, I32, P]),
        "pa_gather_kv": (ctypes.c_int, [D, P, P, P, P, P, I32, P, I32, I32, P]),
        "pa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "pa_last_error_detail": (ctypes.c_char_p, []),
        "pa_version": (ctypes.c_int, []),
        "pa_bench_copy": (ctypes.c_int, [P, P, SZ, P]),
        "pa_bench_read": (ctypes.c_int, [P, SZ, P, P]),
        "pa_bench_flush": (ctypes.c_int, [P, SZ, P]),
        "pa_bench_mfma": (ctypes.c_int, [P, I32, I32, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to libpa must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to libpa must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream, ref):
    if stream is None:
        stream = torch.cuda.current_stream(ref.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status, call):
    if status != 0:
        raise PAError(status, call)


def _need(t, dtype, name, ndim=None):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _shape(t, name, *dims):
    """The kernels trust the sizes they are given: t must be exactly [dims] (None: any size)."""
    if t.dim() != len(dims) or any(d is not None and t.shape[i] != d for i, d in enumerate(dims)):
        want = ", ".join("*" if d is None else str(d) for d in dims)
        raise ValueError(f"{name} must be [{want}], got {list(t.shape)}")


def _pools(desc, k_cache, v_cache):
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache")):
        _shape(t, n, desc.num_blocks, BLOCK_SIZE, desc.num_kv_heads, desc.head_dim)


def _rows(t, name, n, *tail):
    """t is [m, *tail] with m >= n rows (rows past n are neither read nor written)."""
    if t.dim() != 1 + len(tail) or t.shape[0] < n or tuple(t.shape[1:]) != tuple(tail):
        want = ", ".join(str(x) for x in tail)
        raise ValueError(f"{name} must be [>= {n}, {want}], got {list(t.shape)}")


def _table_rows(block_tables, S):
    if block_tables.shape[0] < S:
        raise ValueError(f"block_tables has {block_tables.shape[0]} rows for {S} requests")


def _nbytes(t):
    return t.numel() * t.element_size()


def pa_version() -> int:
    return load().pa_version()


def pa_strerror(status: int) -> str:
    return load().pa_strerror(status).decode()


def pa_last_error_detail() -> str:
    return load().pa_last_error_detail().decode()


def pa_write_kv(desc, key, value, k_cache, v_cache, slot_mapping, stream=None):
    """key/value [N, Hkv, D]; caches [NB, 16, Hkv, D]; slot_mapping int32 [N] (-1 = skip)."""
    dt = torch_dtype(desc)
    for t, n in ((key, "key"), (value, "value"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, dt, n)
    _need(slot_mapping, torch.int32, "slot_mapping", 1)
    n = slot_mapping.numel()
    _pools(desc, k_cache, v_cache)
    _rows(key, "key", n, desc.num_kv_heads, desc.head_dim)
    _rows(value, "value", n, desc.num_kv_heads, desc.head_dim)
    st = load().pa_write_kv(ctypes.byref(desc), _ptr(key), _ptr(value), _ptr(k_cache),
                            _ptr(v_cache), _ptr(slot_mapping), n, _stream(stream, k_cache))
    _check(st, "pa_write_kv")


def pa_decode_partition_tokens(desc, num_seqs, max_context_len) -> int:
    r = load().pa_decode_partition_tokens(ctypes.byref(desc), num_seqs, max_context_len)
    _check(min(r, 0), "pa_decode_partition_tokens")
    return r


def pa_decode_workspace_size(desc, num_seqs, max_context_len, partition_tokens=0) -> int:
    return load().pa_decode_workspace_size(ctypes.byref(desc), num_seqs, max_context_len,
                                           partition_tokens)


def decode_workspace(desc, num_seqs, max_context_len, partition_tokens=0, device="cuda"):
    """A device workspace tensor (uint8) of the size pa_decode needs, or None."""
    n = pa_decode_workspace_size(desc, num_seqs, max_context_len, partition_tokens)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def pa_decode(desc, out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
              scale, workspace=None, partition_tokens=0, stream=None):
    """out/q [S, Hq, D]; block_tables int32 [S, W]; context_lens int32 [S]."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    S = context_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", S, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", S, desc.num_q_heads, desc.head_dim)
    _table_rows(block_tables, S)
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = load().pa_decode(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                          _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S,
                          int(max_context_len), float(scale), int(partition_tokens),
                          _ptr(workspace), ws_bytes, _stream(stream, q))
    _check(st, "pa_decode")


def pa_decode_append(desc, out, q, key, value, k_cache, v_cache, block_tables, context_lens,
                     max_context_len, scale, workspace=None, partition_tokens=0, stream=None):
    """pa_decode after storing each request's newest token (key/value [S, Hkv, D], position
    context_lens[s] - 1, slot from the block table); one kernel pass where possible."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (key, "key"), (value, "value"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    S = context_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", S, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", S, desc.num_q_heads, desc.head_dim)
    _rows(key, "key", S, desc.num_kv_heads, desc.head_dim)
    _rows(value, "value", S, desc.num_kv_heads, desc.head_dim)
    _table_rows(block_tables, S)
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = load().pa_decode_append(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(key), _ptr(value),
                                 _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
                                 _ptr(context_lens), S, int(max_context_len), float(scale),
                                 int(partition_tokens), _ptr(workspace), ws_bytes, _stream(stream, q))
    _check(st, "pa_decode_append")


def pa_decode_append_lean(desc, out, q, key, value, k_cache, v_cache, block_tables, context_lens,
                          max_context_len, scale, workspace=None, stream=None):
    """pa_decode_append (partition_tokens 0) through the low-register decode kernel, for a
    decode that runs beside a chunked prefill on another stream."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (key, "key"), (value, "value"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    S = context_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", S, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", S, desc.num_q_heads, desc.head_dim)
    _rows(key, "key", S, desc.num_kv_heads, desc.head_dim)
    _rows(value, "value", S, desc.num_kv_heads, desc.head_dim)
    _table_rows(block_tables, S)
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = load().pa_decode_append_lean(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(key), _ptr(value),
                                      _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
                                      _ptr(context_lens), S, int(max_context_len), float(scale),
                                      _ptr(workspace), ws_bytes, _stream(stream, q))
    _check(st, "pa_decode_append_lean")


NOALLOC_SCRATCH_BYTES = 64 << 20  # PA_NOALLOC_SCRATCH_BYTES


def pa_decode_append_noalloc(desc, out, q, key, value, k_cache, v_cache, block_tables, context_lens,
                             max_context_len, scale, partition_tokens=0, stream=None):
    """pa_decode_append without a workspace argument: the library's fixed per-GPU scratch
    array holds the split-KV partials (for callers that cannot allocate device memory)."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (key, "key"), (value, "value"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    S = context_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", S, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", S, desc.num_q_heads, desc.head_dim)
    _rows(key, "key", S, desc.num_kv_heads, desc.head_dim)
    _rows(value, "value", S, desc.num_kv_heads, desc.head_dim)
    _table_rows(block_tables, S)
    st = load().pa_decode_append_noalloc(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(key), _ptr(value),
                                         _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
                                         _ptr(context_lens), S, int(max_context_len), float(scale),
                                         int(partition_tokens), _stream(stream, q))
    _check(st, "pa_decode_append_noalloc")


def pa_decode_shared_prefix_workspace_size(desc, num_seqs, max_context_len, prefix_blocks) -> int:
    return load().pa_decode_shared_prefix_workspace_size(ctypes.byref(desc), num_seqs, max_context_len,
                                                         prefix_blocks)


def pa_decode_shared_prefix(desc, out, q, k_cache, v_cache, block_tables, context_lens, max_context_len,
                            prefix_blocks, scale, workspace=None, stream=None):
    """pa_decode when every request's first prefix_blocks table entries are the same blocks;
    the workspace holds pa_decode_shared_prefix_workspace_size bytes."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    S = context_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", S, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", S, desc.num_q_heads, desc.head_dim)
    _table_rows(block_tables, S)
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = load().pa_decode_shared_prefix(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(block_tables), block_tables.shape[1], _ptr(context_lens), S,
                                        int(max_context_len), int(prefix_blocks), float(scale),
                                        _ptr(workspace), ws_bytes, _stream(stream, q))
    _check(st, "pa_decode_shared_prefix")


def pa_prefill_chunk(desc, out, q, k_cache, v_cache, query_start_loc, seq_lens, block_tables,
                     max_query_len, max_seq_len, scale, stream=None):
    """out/q [T, Hq, D]; query_start_loc int32 [S+1]; seq_lens int32 [S]; block_tables [S, W]."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, dt, n)
    for t, n in ((query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        _need(t, torch.int32, n, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    S = seq_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", 0, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", q.shape[0], desc.num_q_heads, desc.head_dim)
    _shape(query_start_loc, "query_start_loc", S + 1)
    _table_rows(block_tables, S)
    st = load().pa_prefill_chunk(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(query_start_loc), _ptr(seq_lens),
                                 _ptr(block_tables), block_tables.shape[1], S, q.shape[0],
                                 int(max_query_len), int(max_seq_len), float(scale),
                                 _stream(stream, q))
    _check(st, "pa_prefill_chunk")


def pa_prefill_chunk_append(desc, out, q, key, value, k_cache, v_cache, query_start_loc, seq_lens,
                            block_tables, max_query_len, max_seq_len, scale, stream=None):
    """pa_prefill_chunk after storing the chunks' new K/V (key/value [T, Hkv, D], row t the
    new token of query row t) into their slots, in one launch."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (key, "key"), (value, "value"), (k_cache, "k_cache"),
                 (v_cache, "v_cache")):
        _need(t, dt, n)
    for t, n in ((query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        _need(t, torch.int32, n, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    S = seq_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", 0, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", q.shape[0], desc.num_q_heads, desc.head_dim)
    _rows(key, "key", q.shape[0], desc.num_kv_heads, desc.head_dim)
    _rows(value, "value", q.shape[0], desc.num_kv_heads, desc.head_dim)
    _shape(query_start_loc, "query_start_loc", S + 1)
    _table_rows(block_tables, S)
    st = load().pa_prefill_chunk_append(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(key), _ptr(value),
                                        _ptr(k_cache), _ptr(v_cache), _ptr(query_start_loc), _ptr(seq_lens),
                                        _ptr(block_tables), block_tables.shape[1], S, q.shape[0],
                                        int(max_query_len), int(max_seq_len), float(scale), _stream(stream, q))
    _check(st, "pa_prefill_chunk_append")


def pa_prefill_chunk_short_max_query_len(desc) -> int:
    st = load().pa_prefill_chunk_short_max_query_len(ctypes.byref(desc))
    _check(min(st, 0), "pa_prefill_chunk_short_max_query_len")
    return st


def pa_prefill_chunk_short_workspace_size(desc, num_seqs, max_query_len) -> int:
    return load().pa_prefill_chunk_short_workspace_size(ctypes.byref(desc), num_seqs, max_query_len)


def chunk_short_workspace(desc, num_seqs, max_query_len, device="cuda"):
    """A device workspace tensor (uint8) of the size pa_prefill_chunk_short needs, or None."""
    n = pa_prefill_chunk_short_workspace_size(desc, num_seqs, max_query_len)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def pa_prefill_chunk_short(desc, out, q, k_cache, v_cache, query_start_loc, seq_lens, block_tables,
                           max_query_len, max_seq_len, scale, workspace, stream=None):
    """pa_prefill_chunk for chunks of at most 16 / (Hq / Hkv) rows, through the decode kernel;
    workspace from chunk_short_workspace."""
    dt = torch_dtype(desc)
    for t, n in ((out, "out"), (q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, dt, n)
    for t, n in ((query_start_loc, "query_start_loc"), (seq_lens, "seq_lens")):
        _need(t, torch.int32, n, 1)
    _need(block_tables, torch.int32, "block_tables", 2)
    S = seq_lens.numel()
    _pools(desc, k_cache, v_cache)
    _rows(q, "q", 0, desc.num_q_heads, desc.head_dim)
    _rows(out, "out", q.shape[0], desc.num_q_heads, desc.head_dim)
    _shape(query_start_loc, "query_start_loc", S + 1)
    _table_rows(block_tables, S)
    ws_bytes = _nbytes(workspace) if workspace is not None else 0
    st = load().pa_prefill_chunk_short(ctypes.byref(desc), _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(query_start_loc), _ptr(seq_lens), _ptr(block_tables),
                                       block_tables.shape[1], S, q.shape[0], int(max_query_len),
                                       int(max_seq_len), float(scale), _ptr(workspace), ws_bytes,
                                       _stream(stream, q))
    _check(st, "pa_prefill_chunk_short")


def pa_copy_blocks(desc, k_cache, v_cache, block_pairs, stream=None):
    """block_pairs int32 [n, 2]: (source block, destination block) per row."""
    dt = torch_dtype(desc)
    _need(k_cache, dt, "k_cache")
    _need(v_cache, dt, "v_cache")
    _need(block_pairs, torch.int32, "block_pairs", 2)
    _pools(desc, k_cache, v_cache)
    _shape(block_pairs, "block_pairs", None, 2)
    st = load().pa_copy_blocks(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(block_pairs),
                               block_pairs.shape[0], _stream(stream, k_cache))
    _check(st, "pa_copy_blocks")


PA_SWAP_OUT = 0
PA_SWAP_IN = 1


def pa_swap_blocks(desc, k_cache, v_cache, host_k, host_v, block_pairs, direction, stream=None):
    """host_k/host_v: pinned CPU tensors [NH, 16, Hkv, D]; block_pairs int32 [n, 2] on the GPU:
    (device, host) for PA_SWAP_OUT, (host, device) for PA_SWAP_IN."""
    dt = torch_dtype(desc)
    for t, n in ((k_cache, "k_cache"), (v_cache, "v_cache"), (host_k, "host_k"), (host_v, "host_v")):
        _need(t, dt, n)
    if host_k.is_cuda or host_v.is_cuda or not host_k.is_pinned() or not host_v.is_pinned():
        raise ValueError("host_k/host_v must be pinned CPU tensors")
    if host_k.shape != host_v.shape or not host_k.is_contiguous() or not host_v.is_contiguous():
        raise ValueError("host_k/host_v must be contiguous and of one shape")
    _pools(desc, k_cache, v_cache)
    _shape(host_k, "host_k", None, BLOCK_SIZE, desc.num_kv_heads, desc.head_dim)
    _need(block_pairs, torch.int32, "block_pairs", 2)
    _shape(block_pairs, "block_pairs", None, 2)
    st = load().pa_swap_blocks(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache),
                               ctypes.c_void_p(host_k.data_ptr()), ctypes.c_void_p(host_v.data_ptr()),
                               host_k.shape[0], _ptr(block_pairs), block_pairs.shape[0], int(direction),
                               _stream(stream, k_cache))
    _check(st, "pa_swap_blocks")


def pa_gather_kv(desc, dst_k, dst_v, k_cache, v_cache, block_tables, context_lens,
                 max_context_len, stream=None):
    """dst_k/dst_v [S, max_context_len, Hkv, D]: each request's logical K/V rows."""
    dt = torch_dtype(desc)
    for t, n in ((dst_k, "dst_k"), (dst_v, "dst_v"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _need(t, dt, n)
    _need(block_tables, torch.int32, "block_tables", 2)
    _need(context_lens, torch.int32, "context_lens", 1)
    S = context_lens.numel()
    _pools(desc, k_cache, v_cache)
    for t, n in ((dst_k, "dst_k"), (dst_v, "dst_v")):
        _shape(t, n, S, int(max_context_len), desc.num_kv_heads, desc.head_dim)
    _table_rows(block_tables, S)
    st = load().pa_gather_kv(ctypes.byref(desc), _ptr(dst_k), _ptr(dst_v), _ptr(k_cache),
                             _ptr(v_cache), _ptr(block_tables), block_tables.shape[1],
                             _ptr(context_lens), context_lens.numel(), int(max_context_len),
                             _stream(stream, k_cache))
    _check(st, "pa_gather_kv")


def pa_bench_copy(dst, src, nbytes, stream=None):
    if nbytes > min(_nbytes(dst), _nbytes(src)):
        raise ValueError("nbytes exceeds a buffer")
    _check(load().pa_bench_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream, src)), "pa_bench_copy")


def pa_bench_read(src, nbytes, sink, stream=None):
    if nbytes > _nbytes(src) or _nbytes(sink) < 4096 * 4:
        raise ValueError("nbytes exceeds src, or sink holds fewer than 4096 floats")
    _check(load().pa_bench_read(_ptr(src), nbytes, _ptr(sink), _stream(stream, src)), "pa_bench_read")


def pa_bench_flush(buf, nbytes, stream=None):
    if nbytes > _nbytes(buf):
        raise ValueError("nbytes exceeds buf")
    _check(load().pa_bench_flush(_ptr(buf), nbytes, _stream(stream, buf)), "pa_bench_flush")


def pa_bench_mfma(operands, workgroups, iters, sink, stream=None):
    """operands: bf16 values, at least workgroups * 512 * 64 of them; sink: workgroups * 512 floats."""
    if _nbytes(operands) < workgroups * 512 * 128 or _nbytes(sink) < workgroups * 512 * 4:
        raise ValueError("operands or sink too small for this many workgroups")
    _check(load().pa_bench_mfma(_ptr(operands), int(workgroups), int(iters), _ptr(sink),
                                _stream(stream, operands)), "pa_bench_mfma")
