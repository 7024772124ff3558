"""One decode step for a fixed batch of running requests, pipelined.

Each step reserves one slot per request (``pa_append_slots``, host), stores
the step's new K/V (``pa_reshape_and_cache``, or its FP8 form for FP8
pools), refreshes the device block tables (``pa_block_tables``) and attends
(``pa_paged_attention_decode`` / ``_fp8``), all enqueued on one stream (the
scheduler loop of ta-paperlens: blocks are reserved for every running
request before the step's forward pass).  The step's slots, lengths and
work list sit in one pinned host buffer; the block table stays in device
memory and only its entries that changed since the previous step (a request
that took a new block, a copy-on-write replacement) travel, as (index,
value) pairs, so one ``pa_stage_update`` launch on the step's stream moves
both.  The first step, or one that changes more entries than the update
list holds, copies the whole table.  Measured per config-3 step before the
update list: the runtime's copy from pinned memory (several launches)
262 us, one ``pa_stage_copy`` of the whole padded table 250 us, the kernels
reading the pinned buffer in place 249 us but with the decode kernel itself
~10 us slower (its table reads cross the host link); that copy on a second
stream, overlapping the previous step and waited for by events, 253 vs
249 us serial.  Host buffers are used round-robin: the host fills buffer
i+1 while the GPU still runs step i.
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
        # one int32 staging layout in pinned host memory: slots, lengths and
        # work list (copied every step, so they come first and the work list
        # last: a step copies only the entries it uses), then table updates
        # ((index, value) pairs), then a whole table for full uploads; each
        # section starts on a 64-byte boundary
        p_cap = -(-self.max_len_cap // self.partition)
        up = lambda n: -(-n // 16) * 16
        n_tab = self.B * self.max_blocks
        self.upd_cap = max(1024, 4 * self.B)
        self.o_len = up(self.B)
        self.o_items = self.o_len + up(self.B)
        self.o_upd = up(self.o_items + self.B * p_cap)
        self.o_full = self.o_upd + up(2 * self.upd_cap)
        total = self.o_full + up(n_tab)
        self.h_buf = [torch.empty(total, dtype=torch.int32, pin_memory=True) for _ in range(depth)]
        self.h_dev = [L.pa_host_device_pointer(b) for b in self.h_buf]
        self.d_buf = torch.empty(self.o_upd, dtype=torch.int32, device=dev)
        self.d_slots = self.d_buf[:self.B]
        self.d_len = self.d_buf[self.o_len:self.o_len + self.B]
        self.d_items = self.d_buf[self.o_items:]
        # the device block table, and what the launches enqueued so far leave
        # in it (None: nothing yet)
        self.d_tab_buf = torch.empty(up(n_tab), dtype=torch.int32, device=dev)
        self.d_tab = self.d_tab_buf[:n_tab].view(self.B, self.max_blocks)
        self.shadow: Optional[np.ndarray] = None
        self.full_uploads = 0
        self.updated_entries = 0
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
        n_tab = self.B * self.max_blocks
        tab_np = h[self.o_full:self.o_full + n_tab]
        len_np = h[self.o_len:self.o_len + self.B]
        L.pa_block_tables(self.cache.pool, self.ids, self.max_blocks,
                          tables=tab_np.reshape(self.B, self.max_blocks), lens=len_np)
        max_len = int(len_np.max())
        if max_len > self.max_len_cap:
            raise ValueError("a request outgrew the stepper's max_len_cap")
        self.last_lens = len_np.copy()
        n_items = len(L.pa_decode_work_items(len_np, self.partition, out=h[self.o_items:]))
        nbytes = -(-(self.o_items + n_items) // 4) * 16  # whole 16-byte chunks
        changed = None
        if self.shadow is not None:
            changed = np.flatnonzero(tab_np != self.shadow)
            if len(changed) > self.upd_cap:
                changed = None
        with torch.cuda.stream(stream):
            if changed is None:
                # whole table (16-byte chunks; the device buffer is padded)
                L.pa_stage_copy(self.h_dev[r] + 4 * self.o_full, self.d_tab_buf,
                                4 * self.d_tab_buf.numel(), stream)
                L.pa_stage_copy(self.h_dev[r], self.d_buf, nbytes, stream)
                self.shadow = tab_np.copy()
                self.full_uploads += 1
            else:
                n_upd = len(changed)
                upd = h[self.o_upd:self.o_upd + 2 * n_upd].reshape(n_upd, 2)
                upd[:, 0] = changed
                upd[:, 1] = tab_np[changed]
                L.pa_stage_update(self.h_dev[r], self.d_buf, nbytes,
                                  self.h_dev[r] + 4 * self.o_upd, n_upd, self.d_tab, n_tab,
                                  stream)
                self.shadow[changed] = tab_np[changed]
                self.updated_entries += n_upd
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
