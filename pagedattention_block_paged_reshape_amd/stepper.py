"""One decode step for a fixed batch of running requests, pipelined.

Each step reserves one slot per request (``pa_append_slots``, host), stores
the step's new K/V (``pa_reshape_and_cache``, or its FP8 form for FP8
pools), refreshes the device block tables (``pa_block_tables``) and attends
(``pa_paged_attention_decode`` / ``_fp8``), all enqueued on one stream (the
scheduler loop of ta-paperlens: blocks are reserved for every running
request before the step's forward pass).  The step's slots, tables, lengths
and work list sit in one pinned host buffer and go to device memory in one
``pa_stage_copy`` launch on the step's stream.  Measured per config-3 step:
the runtime's copy from pinned memory (several launches) 262 us, this copy
250 us, the kernels reading the pinned buffer in place 249 us but with the
decode kernel itself ~10 us slower (its table reads cross the host link);
this copy on a second stream, overlapping the previous step and waited for
by events, 253 vs 249 us serial.  Host buffers are used round-robin: the
host fills buffer i+1 while the GPU still runs step i.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import _lib as L
from .cache import DEFAULT_PARTITION, PagedKVCache


class DecodeStepper:
    def __init__(self, cache: PagedKVCache, seq_ids, num_q_heads: int, scale: float,
                 max_len_cap: int, partition: int = DEFAULT_PARTITION, depth: int = 3):
        self.cache = cache
        self.ids = np.ascontiguousarray(np.asarray(seq_ids, dtype=np.int64))
        self.B = len(self.ids)
        self.ones = np.ones(self.B, dtype=np.int32)
        self.n_q, self.scale, self.partition = int(num_q_heads), float(scale), int(partition)
        self.max_len_cap = int(max_len_cap)
        self.max_blocks = -(-self.max_len_cap // L.BLOCK_SIZE)
        dev = cache.device
        self.depth = depth
        # one int32 staging layout, host and device: slots, tables, lengths,
        # work list (each section starting on a 64-byte boundary; the work
        # list last, so a step copies only the entries it uses)
        p_cap = -(-self.max_len_cap // self.partition)
        up = lambda n: -(-n // 16) * 16
        self.o_tab = up(self.B)
        self.o_len = self.o_tab + up(self.B * self.max_blocks)
        self.o_items = self.o_len + up(self.B)
        total = up(self.o_items + self.B * p_cap)
        self.h_buf = [torch.empty(total, dtype=torch.int32, pin_memory=True) for _ in range(depth)]
        self.h_dev = [L.pa_host_device_pointer(b) for b in self.h_buf]
        self.d_buf = torch.empty(total, dtype=torch.int32, device=dev)
        self.d_slots = self.d_buf[:self.B]
        self.d_tab = self.d_buf[self.o_tab:self.o_tab + self.B * self.max_blocks].view(
            self.B, self.max_blocks)
        self.d_len = self.d_buf[self.o_len:self.o_len + self.B]
        self.d_items = self.d_buf[self.o_items:]
        # event r: the copy out of host buffer r has completed
        self.done = [torch.cuda.Event() for _ in range(depth)]
        self.used = [False] * depth
        self.ws_bytes = L.pa_decode_workspace_bytes(self.B, self.n_q, cache.d, self.max_len_cap,
                                                    self.partition)
        self.workspace = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8, device=dev)
        self.out = torch.empty((self.B, self.n_q, cache.d), dtype=torch.float16, device=dev)
        self.i = 0
        self.last_lens: Optional[np.ndarray] = None

    def step(self, q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
             stream: Optional[torch.cuda.Stream] = None, events=None) -> torch.Tensor:
        """Enqueue one step.  ``events``: optional dict of (start, end) event
        pairs named 'cache' and 'decode' recorded around those launches."""
        stream = stream or torch.cuda.current_stream(self.cache.device)
        r = self.i % self.depth
        if self.used[r]:
            self.done[r].synchronize()          # host buffer r has been copied out
        h = self.h_buf[r].numpy()
        slots_np = h[:self.B]
        _, copies = L.pa_append_slots(self.cache.pool, self.ids, self.ones, slots_out=slots_np)
        tab_np = h[self.o_tab:self.o_tab + self.B * self.max_blocks].reshape(self.B, self.max_blocks)
        len_np = h[self.o_len:self.o_len + self.B]
        L.pa_block_tables(self.cache.pool, self.ids, self.max_blocks, tables=tab_np, lens=len_np)
        max_len = int(len_np.max())
        if max_len > self.max_len_cap:
            raise ValueError("a request outgrew the stepper's max_len_cap")
        self.last_lens = len_np.copy()
        n_items = len(L.pa_decode_work_items(len_np, self.partition, out=h[self.o_items:]))
        nbytes = -(-(self.o_items + n_items) // 4) * 16  # whole 16-byte chunks
        with torch.cuda.stream(stream):
            L.pa_stage_copy(self.h_dev[r], self.d_buf, nbytes, stream)
            self.done[r].record(stream)
            self.used[r] = True
            if events is not None:
                events["cache"][0].record(stream)
            if len(copies):
                d_copies = torch.from_numpy(np.ascontiguousarray(copies)).to(self.cache.device)
                self.cache.copy_blocks(d_copies, len(copies), stream)
            self.cache.store(k_new, v_new, self.d_slots, self.B, stream)
            if events is not None:
                events["cache"][1].record(stream)
                events["decode"][0].record(stream)
            flags = L.PA_DECODE_KEEP_KV if self.cache.shares_blocks() else 0
            self.cache.decode(self.out, q, self.d_tab, self.max_blocks, self.d_len, self.B,
                              self.n_q, self.scale, self.partition, max_len, self.d_items,
                              n_items, self.workspace, self.ws_bytes, stream, flags=flags)
            if events is not None:
                events["decode"][1].record(stream)
        self.i += 1
        return self.out
