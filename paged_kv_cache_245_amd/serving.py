"""One continuous-batching step on the GPU, from a host scheduler's batch.

A step (arcyou teardown of vLLM paged attention, "Continuous batching: rebuild
the batch every step") mixes prompt chunks and single generated tokens. Given
the batch that libpa_host.so's scheduler planned (host.Scheduler.schedule) and
the block operations the pool queued for it (host.BlockPool.take_ops), this
module issues, on the caller's stream: the block operations in their order
(pa_copy_blocks for copy-on-write copies, pa_swap_blocks for swap-outs and
swap-ins, consecutive operations of one kind batched into one call when none
writes a block another reads or writes), one copy of the step's metadata to
the GPU, pa_write_kv for the K/V of the requests given more than one token,
pa_prefill_chunk for those requests, and pa_decode_append for the ones given
exactly one (their new K/V is stored by the decode itself). When a step has
both, the decode runs on a second stream (default priority) forked after the
write and joined before the step returns, through pa_decode_append_lean, whose
wavefronts fit beside the prefill's on every compute unit: the prefill keeps
the matrix cores busy while the decode streams K/V from HBM. The two calls
touch disjoint memory (the decode stores only into each one-token request's
own last block; blocks shared with other requests are full and never
written). Short chunks (at most 16 / (q heads per kv head) tokens, as when a
request scores its draft tokens) go through pa_prefill_chunk_short: the
scheduler lists the multi-token requests longest first, so the short ones end
the group, and the call takes them after the pa_prefill_chunk of the rest, on
the caller's stream. A step whose chunks are all short runs that call and then
the decode on the caller's stream: both stream K/V from HBM, and running them
side by side gains nothing. Marshalling and sequencing only; the work runs in
libpa.so's kernels.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as pa
from .host import OP_COPY, OP_SWAP_IN, OP_SWAP_OUT


def batch_ops(ops):
    """Split ordered block operations into runs of one kind that may execute as one call:
    a run ends where an operation would write a block that the run already reads or
    writes, or read a block that the run writes. Returns [(kind, [(src, dst), ...])]."""
    runs = []
    for kind, src, dst in ops:
        # a block is named by (memory, id); copies live on the device, swaps cross to the host
        s_mem, d_mem = {OP_COPY: ("d", "d"), OP_SWAP_OUT: ("d", "h"), OP_SWAP_IN: ("h", "d")}[kind]
        s_key, d_key = (s_mem, src), (d_mem, dst)
        if runs and runs[-1][0] == kind:
            reads, writes = runs[-1][2], runs[-1][3]
            if d_key not in reads and d_key not in writes and s_key not in writes:
                runs[-1][1].append((src, dst))
                reads.add(s_key)
                writes.add(d_key)
                continue
        runs.append([kind, [(src, dst)], {s_key}, {d_key}])
    return [(kind, pairs) for kind, pairs, _, _ in runs]


def short_tail_start(counts, short_rows):
    """Index of the first multi-token request whose chunk goes to pa_prefill_chunk_short:
    0 when every chunk has at most short_rows rows, the start of the short tail when the
    counts come longest first (the scheduler's order), else len(counts) (none)."""
    counts = np.asarray(counts)
    P = len(counts)
    short = counts <= short_rows
    if P and short.all():
        return 0
    if P and short[-1] and np.all(np.diff(counts) <= 0):
        return int(np.argmax(short))
    return P


class StepRunner:
    """Device buffers for the steps of one pool: metadata staging and the decode workspace.

    Metadata goes through two pinned host buffers used in turn; before one is
    refilled, the copy that last read it is waited for, so the host can plan the
    next step while the GPU runs the previous one.
    """

    def __init__(self, desc, k_cache, v_cache, scale, max_seqs, max_tokens, max_blocks_per_seq,
                 device="cuda", host_k=None, host_v=None, side_stream=None):
        """host_k/host_v: the pinned CPU swap space [num_host_blocks, 16, Hkv, D], if any.
        side_stream: the stream for the decode beside the prefill (default: a new one). The
        two overlap only if HIP put this stream on another hardware queue than the caller's;
        it hands out GPU_MAX_HW_QUEUES (4 by default) queues to streams, so a stream
        created early in the process, among the first few, normally has its own."""
        self.desc, self.k, self.v, self.scale = desc, k_cache, v_cache, float(scale)
        self.host_k, self.host_v = host_k, host_v
        self.max_seqs, self.max_tokens, self.max_blocks = max_seqs, max_tokens, max_blocks_per_seq
        self.device = torch.device(device)
        # room for one step's metadata (int32): qsl | seq_lens | tables | slots | the short
        # chunks' own qsl
        self.n_meta = (max_seqs + 1) + max_seqs + max_seqs * max_blocks_per_seq + max_tokens + (max_seqs + 1)
        self.host = [torch.empty(self.n_meta, dtype=torch.int32, pin_memory=True) for _ in range(2)]
        self.done = [None, None]
        self.turn = 0
        self.meta = torch.empty(self.n_meta, dtype=torch.int32, device=self.device)
        self.ws = pa.decode_workspace(desc, max_seqs, max_blocks_per_seq * 16, 0, self.device)
        self.ws_bytes = 0 if self.ws is None else self.ws.numel()
        # steps of short chunks: pa_prefill_chunk_short and its own workspace
        self.short_rows = 0
        self.ws_short = None
        self.short_steps = 0  # steps with chunks through pa_prefill_chunk_short
        self.split_steps = 0  # of them, steps that also had longer chunks
        if desc.dtype == pa.PA_BF16 and max_seqs <= 8192:
            self.short_rows = pa.pa_prefill_chunk_short_max_query_len(desc)
            self.ws_short = pa.chunk_short_workspace(desc, max_seqs, self.short_rows, self.device)
        # default priority, like every stream here
        self.side = side_stream if side_stream is not None else torch.cuda.Stream(self.device)

    def run_ops(self, ops):
        """The pool's block operations (kind, source, destination), in order."""
        for kind, pairs in batch_ops(ops):
            t = torch.tensor(np.asarray(pairs, dtype=np.int32).reshape(-1, 2), device=self.device)
            if kind == OP_COPY:
                pa.pa_copy_blocks(self.desc, self.k, self.v, t)
            else:
                if self.host_k is None:
                    raise ValueError("swap operations need the host swap space")
                pa.pa_swap_blocks(self.desc, self.k, self.v, self.host_k, self.host_v, t,
                                  pa.PA_SWAP_OUT if kind == OP_SWAP_OUT else pa.PA_SWAP_IN)

    def run(self, batch, q, key, value, out, ops=()):
        """q/out [N, Hq, D], key/value [N, Hkv, D]: the step's new tokens in batch order;
        ops: the block operations the pool queued while the step was planned."""
        self.run_ops(ops)
        S, N, P = batch.num_seqs, batch.num_tokens, batch.num_prefills
        if S == 0:
            return
        mb = batch.block_tables.shape[1]
        if S > self.max_seqs or N > self.max_tokens or mb > self.max_blocks:
            raise ValueError("step larger than the buffers of this StepRunner")
        stream = torch.cuda.current_stream(self.device)

        # pack the metadata (qsl | seq_lens | tables | slots) into the next pinned buffer,
        # then one host-to-device copy of the used length
        buf = self.host[self.turn]
        if self.done[self.turn] is not None:
            self.done[self.turn].synchronize()
        h = buf.numpy()
        o_seq = P + 1
        o_tab = o_seq + S
        o_slot = o_tab + S * mb
        end = o_slot + N
        h[:o_seq] = batch.query_start_loc
        h[o_seq:o_tab] = batch.seq_lens
        h[o_tab:o_slot] = batch.block_tables.reshape(-1)
        h[o_slot:end] = batch.slot_mapping
        # multi-token requests come longest first (the scheduler's order): those from j on
        # are short chunks. A batch in another order goes through pa_prefill_chunk whole
        # unless every chunk is short.
        counts = batch.counts[:P]
        j = short_tail_start(counts, self.short_rows)
        o_short = end
        if j < P:  # their row offsets, from 0 at their first row
            end = o_short + (P - j) + 1
            h[o_short:end] = batch.query_start_loc[j:] - batch.query_start_loc[j]
        self.meta[:end].copy_(buf[:end], non_blocking=True)
        ev = torch.cuda.Event()
        ev.record(stream)
        self.done[self.turn] = ev
        self.turn ^= 1

        qsl = self.meta[:o_seq]
        seq = self.meta[o_seq:o_tab]
        tables = self.meta[o_tab:o_slot].view(S, mb)
        slots = self.meta[o_slot:o_short]
        n_pf = int(batch.query_start_loc[-1])
        if S > P:
            need = pa.pa_decode_workspace_size(self.desc, S - P, int(batch.seq_lens[P:].max()))
            if need > self.ws_bytes:
                raise ValueError("decode workspace too small for this step")
        short = P > 0 and j == 0  # every chunk short
        fork = P > 0 and S > P and not short
        if P:
            pa.pa_write_kv(self.desc, key[:n_pf], value[:n_pf], self.k, self.v, slots[:n_pf])
            if fork:
                self.side.wait_stream(stream)
            if j > 0:  # the longer chunks on the matrix cores
                r = int(batch.query_start_loc[j])
                pa.pa_prefill_chunk(self.desc, out[:r], q[:r], self.k, self.v, qsl[:j + 1], seq[:j], tables[:j],
                                    int(counts[0]), int(batch.seq_lens[:j].max()), self.scale)
            if j < P:  # the short ones through the decode kernel
                r = int(batch.query_start_loc[j])
                self.short_steps += 1
                self.split_steps += j > 0
                pa.pa_prefill_chunk_short(self.desc, out[r:n_pf], q[r:n_pf], self.k, self.v,
                                          self.meta[o_short:o_short + P - j + 1], seq[j:P], tables[j:P],
                                          int(counts[j]), int(batch.seq_lens[j:P].max()), self.scale,
                                          self.ws_short)
        if S > P:
            # a one-token request's new token is its newest, at position seq_len - 1
            args = (self.desc, out[n_pf:N], q[n_pf:N], key[n_pf:N], value[n_pf:N], self.k, self.v,
                    tables[P:], seq[P:], int(batch.seq_lens[P:].max()), self.scale, self.ws)
            if fork:
                pa.pa_decode_append_lean(*args, stream=self.side)
                stream.wait_stream(self.side)
            else:
                pa.pa_decode_append(*args, stream=stream)
