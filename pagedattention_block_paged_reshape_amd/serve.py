"""Multi-step serving loop: the C++ scheduler (pa_sched_*) plans each step,
and this loop runs the step's kernels on the GPU.

Per step ([lens] "scheduler skeleton": admit, step all running requests,
retire finished ones, preempt when out of blocks; [ngrok] scheduler section):
  1. pa_sched_schedule: chunks (request, first position, length) within the
     token budget, decode first, their KV slots, and any preemptions;
  2. the step's new K/V rows (a synthetic model: rows are a fixed function of
     request and position, see synth.serving) go to their slots with
     pa_reshape_and_cache;
  3. decode chunks (one new token each) attend their requests' whole
     sequences in one pa_paged_attention_decode launch; prefill chunks each
     get a pa_paged_attention_prefill launch (causal over the cache);
  4. pa_sched_commit retires finished requests and frees their blocks.
With swap=True the scheduler preempts by swapping ([lens] skeleton: move
the request to CPU memory instead of recomputing it): before anything else
in a step, this loop copies the K/V of requests swapped out to pinned host
memory and writes those of resumed requests back into their new blocks.
With mixed=True a step with both kinds of work runs its decode batch and its
first prefill chunk in one pa_paged_attention_mixed launch (bitwise the same
outputs as the two separate launches).
This module only marshals arguments and launches; every step of the path
runs in the library.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

from . import _lib as L
from .cache import PagedKVCache


class ServingLoop:
    def __init__(self, cache: PagedKVCache, num_q_heads: int, scale: float, token_budget: int,
                 max_running: int, partition: int = 512, row_fn=None,
                 keep_outputs: bool = False, rows_fn=None, swap: bool = False,
                 mixed: bool = False):
        """row_fn(req, pos, tag, width) -> fp16 rows on the cache's device
        (int64 device tensors in), or rows_fn(req, pos, width_kv, width_q) ->
        (k, v, q) rows in one call; keep_outputs stores every attention
        output row by (request, position) for checking."""
        self.cache = cache
        self.n_q = int(num_q_heads)
        self.scale = float(scale)
        self.budget = int(token_budget)
        self.max_running = int(max_running)
        self.partition = int(partition)
        self.row_fn = row_fn
        self.rows_fn = rows_fn
        self.keep = keep_outputs
        # (request, position) -> (output row [n_q][d], "decode" | "prefill")
        self.outputs: Dict[Tuple[int, int], Tuple[torch.Tensor, str]] = {}
        self.sched = L.pa_sched_create(cache.pool, self.budget, self.max_running)
        self.swap = bool(swap)
        self.mixed = bool(mixed)
        if self.swap:
            L.pa_sched_set_swap(self.sched, True)
        self.saved: Dict[int, Tuple[torch.Tensor, torch.Tensor]] = {}  # swapped-out K/V
        dev = cache.device
        self.d = cache.d
        self.stats = {"steps": 0, "decode_tokens": 0, "prefill_tokens": 0, "preempted": 0,
                      "finished": 0, "swapped_out": 0, "swapped_in": 0, "mixed_launches": 0}
        self._ws = torch.zeros(16, dtype=torch.uint8, device=dev)
        self._pws = torch.zeros(16, dtype=torch.uint8, device=dev)
        self.dev = dev

    def close(self):
        if self.sched:
            L.pa_sched_destroy(self.sched)
            self.sched = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, req_id: int, prompt_len: int, output_len: int):
        L.pa_sched_add_request(self.sched, req_id, prompt_len, output_len)

    def _workspace(self, attr: str, nbytes: int) -> torch.Tensor:
        ws = getattr(self, attr)
        if ws.numel() < nbytes:
            ws = torch.zeros(nbytes, dtype=torch.uint8, device=self.dev)
            setattr(self, attr, ws)
        return ws

    @staticmethod
    def _hold(stream, *tensors):
        """The launches only keep raw device addresses: tie each tensor to
        the stream the kernels run on, so that the caching allocator does not
        hand its memory out again before that stream's work so far is done
        (the Python references are dropped when this step returns)."""
        for t in tensors:
            if t is not None and t.device.type == "cuda":
                t.record_stream(stream)

    def _h2d(self, a: np.ndarray) -> torch.Tensor:
        """Host array to the device through a pinned staging copy, so the
        copy never waits for the GPU to drain the stream."""
        return torch.from_numpy(np.ascontiguousarray(a)).pin_memory().to(self.dev,
                                                                         non_blocking=True)

    def step(self, stream=None) -> List[int]:
        """Plan and run one step; returns the requests that finished.  All of
        the step's device work (row generation, host-to-device copies,
        allocations and the library's launches) goes to `stream`."""
        stream = stream or torch.cuda.current_stream(self.dev)
        with torch.cuda.stream(stream):
            return self._step(stream)

    def _step(self, stream) -> List[int]:
        plan = L.pa_sched_schedule(self.sched, self.budget, self.max_running)
        items = plan["items"]
        self.stats["preempted"] += len(plan["preempted"])
        if self.swap:
            # outs first: their blocks may already belong to this step's writes
            for rid, kind, _, blocks in L.pa_sched_swaps(self.sched):
                if kind == "out":
                    self.saved[rid] = self.cache.gather_to_host(blocks, stream)
                    self.stats["swapped_out"] += 1
                else:
                    k_host, v_host = self.saved.pop(rid)
                    self.cache.scatter_from_host(blocks, k_host, v_host, stream)
                    self.stats["swapped_in"] += 1
        if items:
            req = np.concatenate([np.full(n, r, dtype=np.int64) for r, _, n, _ in items])
            pos = np.concatenate([np.arange(s, s + n, dtype=np.int64) for _, s, n, _ in items])
            d_req = self._h2d(req)
            d_pos = self._h2d(pos)
            width = self.cache.n_kv * self.d
            if self.rows_fn is not None:
                k, v, q = self.rows_fn(d_req, d_pos, width, self.n_q * self.d)
                k = k.contiguous().view(-1, self.cache.n_kv, self.d)
                v = v.contiguous().view(-1, self.cache.n_kv, self.d)
                q = q.view(-1, self.n_q, self.d)
            else:
                k = self.row_fn(d_req, d_pos, 0, width).view(-1, self.cache.n_kv, self.d)
                v = self.row_fn(d_req, d_pos, 1, width).view(-1, self.cache.n_kv, self.d)
                q = self.row_fn(d_req, d_pos, 2, self.n_q * self.d).view(-1, self.n_q, self.d)
            slots = self._h2d(plan["slots"])
            if len(plan["copies"]):
                d_copies = self._h2d(plan["copies"])
                self.cache.copy_blocks(d_copies, len(plan["copies"]), stream)
                self._hold(stream, d_copies)
            self.cache.store(k, v, slots, len(req), stream)
            self._hold(stream, k, v, slots)
            offs = np.cumsum([0] + [n for _, _, n, _ in items])
            dec = [i for i, it in enumerate(items) if it[3]]
            pre = [i for i, it in enumerate(items) if not it[3]]
            if dec:
                rows = offs[dec]
                # decode items come first (one token each), so their query
                # rows are usually a leading slice
                if np.array_equal(rows, np.arange(len(dec))):
                    q_dec = q[:len(dec)]
                else:
                    q_dec = q[self._h2d(rows.astype(np.int64))]
                first = None
                if self.mixed and pre:
                    first = pre[0]
                    pre = pre[1:]
                    r, s, n, _ = items[first]
                    first = (r, s, n, q[offs[first]:offs[first] + n])
                self._decode([items[i] for i in dec], q_dec, stream, chunk=first)
            for i in pre:
                r, s, n, _ = items[i]
                self._prefill(r, s, n, q[offs[i]:offs[i] + n], stream)
            self.stats["decode_tokens"] += len(dec)
            self.stats["prefill_tokens"] += int(sum(it[2] for it in items if not it[3]))
        done = L.pa_sched_commit(self.sched, self.max_running)
        self.stats["steps"] += 1
        self.stats["finished"] += len(done)
        return done

    def _decode(self, items, q: torch.Tensor, stream, chunk=None):
        """Decode attention for the items; with chunk = (request, start,
        length, query rows) that prefill chunk runs in the same launch."""
        ids = [r for r, _, _, _ in items]
        # each request's length after this step is known from its item
        max_blocks = max(-(-(s + 1) // L.BLOCK_SIZE) for _, s, _, _ in items)
        tab, ln = L.pa_block_tables(self.cache.pool, ids, max_blocks)
        assert [int(x) for x in ln] == [s + 1 for _, s, _, _ in items]
        max_len = int(ln.max())
        work = L.pa_decode_work_items(ln, self.partition)
        ws_bytes = L.pa_decode_workspace_bytes(len(ids), self.n_q, self.d, max_len, self.partition)
        ws = self._workspace("_ws", max(ws_bytes, 16))
        out = torch.empty((len(ids), self.n_q, self.d), dtype=torch.float16, device=self.dev)
        d_tab = self._h2d(tab)
        d_len = self._h2d(ln)
        d_work = self._h2d(work)
        flags = L.PA_DECODE_KEEP_KV if self.cache.shares_blocks() else 0
        # a contiguous copy of the queries (a slice of the step's fused rows
        # is not): bound to a name so it outlives every launch that reads it
        q_c = q.contiguous()
        if chunk is None:
            self.cache.decode(out, q_c, d_tab, max_blocks, d_len, len(ids), self.n_q,
                              self.scale, self.partition, max_len, d_work, len(work), ws,
                              ws_bytes, stream, flags=flags)
            self._hold(stream, q_c, out, d_tab, d_len, d_work, ws)
        else:
            r, s, n, qc = chunk
            pf_blocks = -(-(s + n) // L.BLOCK_SIZE)
            ptab, pln = L.pa_block_tables(self.cache.pool, [r], pf_blocks)
            assert int(pln[0]) == s + n
            qc = qc.contiguous()
            pout = torch.empty((n, self.n_q, self.d), dtype=torch.float16, device=self.dev)
            c_dec = L.decode_batch(out, q_c, d_tab, max_blocks, d_len, len(ids),
                                   self.partition, max_len, d_work, len(work))
            d_ptab = self._h2d(ptab[0])
            c_pf = L.prefill_chunk(pout, qc, d_ptab, pf_blocks, s, n)
            mws_bytes = L.pa_mixed_workspace_bytes(c_dec, c_pf, self.n_q, self.d)
            mws = self._workspace("_ws", max(mws_bytes, 16))
            L.pa_paged_attention_mixed(c_dec, c_pf, self.cache.kv, self.n_q, self.scale, mws,
                                       mws_bytes, stream, flags=flags)
            self._hold(stream, q_c, out, d_tab, d_len, d_work, qc, pout, d_ptab, mws)
            self.stats["mixed_launches"] += 1
            if self.keep:
                kept = pout.clone()
                for j in range(n):
                    self.outputs[(r, s + j)] = (kept[j], "prefill")
        if self.keep:
            # copies: the launch buffers go back to the allocator as they would
            # without keep_outputs
            kept = out.clone()
            for j, (r, s, _, _) in enumerate(items):
                self.outputs[(r, s)] = (kept[j], "decode")

    def _prefill(self, r: int, s: int, n: int, q: torch.Tensor, stream):
        max_blocks = -(-(s + n) // L.BLOCK_SIZE)
        tab, ln = L.pa_block_tables(self.cache.pool, [r], max_blocks)
        assert int(ln[0]) == s + n
        ws_bytes = L.pa_prefill_workspace_bytes(n, self.n_q, self.d, s)
        ws = self._workspace("_pws", max(ws_bytes, 16))
        out = torch.empty((n, self.n_q, self.d), dtype=torch.float16, device=self.dev)
        d_tab = self._h2d(tab[0])
        q_c = q.contiguous()
        L.pa_paged_attention_prefill(out, q_c, self.cache.kv, d_tab, max_blocks, s, n,
                                     self.n_q, self.scale, ws, ws_bytes, stream)
        self._hold(stream, q_c, out, d_tab, ws)
        if self.keep:
            kept = out.clone()
            for j in range(n):
                self.outputs[(r, s + j)] = (kept[j], "prefill")

    def request(self, req_id: int):
        """(computed input tokens, generated tokens, preemptions)."""
        return L.pa_sched_request(self.sched, req_id)

    def sched_stats(self) -> dict:
        return L.pa_sched_get_stats(self.sched)
