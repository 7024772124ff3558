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
A step's host-built arrays (request ids and positions of its rows, slots,
copy-on-write list, block tables, lengths, work lists) are packed into one
pinned staging buffer and moved to the device by one pa_stage_copy launch.
This module only marshals arguments and launches; every step of the path
runs in the library.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np
import torch

from . import _lib as L
from .cache import PagedKVCache


class _Staging:
    """A ring of pinned host buffers and one device buffer: a step's arrays
    are packed into the next host buffer (16-byte aligned sections) and moved
    by one pa_stage_copy launch; the host waits for a buffer's copy before
    packing it again."""

    def __init__(self, dev, nbytes: int = 1 << 16, depth: int = 3):
        self.dev = dev
        self.depth = depth
        self.host = [self._pinned(nbytes) for _ in range(depth)]
        self.done = [torch.cuda.Event() for _ in range(depth)]
        self.used = [False] * depth
        self.d_buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.r = -1
        self.off = 0
        self.secs: List[Tuple[int, int, np.dtype]] = []

    @staticmethod
    def _pinned(nbytes: int):
        buf = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        return buf, L.pa_host_device_pointer(buf)

    def begin(self) -> None:
        self.r = (self.r + 1) % self.depth
        if self.used[self.r]:
            self.done[self.r].synchronize()
        self.off = 0
        self.secs = []

    def add(self, a: np.ndarray) -> int:
        """Pack `a`; returns its section index."""
        a = np.ascontiguousarray(a)
        n = a.nbytes
        buf, _ = self.host[self.r]
        if self.off + n > buf.numel():
            grown = self._pinned(max(2 * buf.numel(), -(-(self.off + n) // 4096) * 4096 * 2))
            grown[0][:self.off].copy_(buf[:self.off])
            self.host[self.r] = grown
            buf = grown[0]
        if n:
            buf.numpy()[self.off:self.off + n] = a.view(np.uint8).reshape(-1)
        self.secs.append((self.off, a.size, a.dtype))
        self.off += -(-n // 16) * 16
        return len(self.secs) - 1

    def upload(self, stream) -> List[torch.Tensor]:
        """One copy of the packed sections; returns their device views."""
        if self.d_buf.numel() < self.off:
            self.d_buf = torch.empty(2 * self.off, dtype=torch.uint8, device=self.dev)
        if self.off:
            L.pa_stage_copy(self.host[self.r][1], self.d_buf, self.off, stream)
        self.done[self.r].record(stream)
        self.used[self.r] = True
        tdt = {np.dtype(np.int32): torch.int32, np.dtype(np.int64): torch.int64}
        return [self.d_buf[o:o + n * np.dtype(dt).itemsize].view(tdt[np.dtype(dt)])
                for o, n, dt in self.secs]


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
        self.stage = _Staging(dev)

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
            offs = np.cumsum([0] + [n for _, _, n, _ in items])
            dec = [i for i, it in enumerate(items) if it[3]]
            pre = [i for i, it in enumerate(items) if not it[3]]
            first = None
            if self.mixed and dec and pre:
                first, pre = pre[0], pre[1:]
            # every array the step's launches read, packed and moved at once
            st = self.stage
            st.begin()
            i_req, i_pos = st.add(req), st.add(pos)
            i_slots = st.add(plan["slots"])
            i_copies = st.add(plan["copies"]) if len(plan["copies"]) else None
            dec_host = self._decode_host([items[i] for i in dec]) if dec else None
            rows = offs[dec] if dec else None
            lead = dec and np.array_equal(rows, np.arange(len(dec)))
            i_rows = st.add(rows.astype(np.int64)) if dec and not lead else None
            i_dec = [st.add(a) for a in dec_host[:3]] if dec else None
            pf_host = {i: self._prefill_host(*items[i][:3]) for i in ([first] if first is not None
                                                                      else []) + pre}
            i_pf = {i: st.add(h[0]) for i, h in pf_host.items()}
            dv = st.upload(stream)

            d_req, d_pos = dv[i_req], dv[i_pos]
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
            if i_copies is not None:
                self.cache.copy_blocks(dv[i_copies], len(plan["copies"]), stream)
            self.cache.store(k, v, dv[i_slots], len(req), stream)
            self._hold(stream, k, v)
            if dec:
                # decode items come first (one token each), so their query
                # rows are usually a leading slice
                q_dec = q[:len(dec)] if lead else q[dv[i_rows]]
                chunk = None
                if first is not None:
                    r, s, n, _ = items[first]
                    chunk = (r, s, n, q[offs[first]:offs[first] + n], pf_host[first],
                             dv[i_pf[first]])
                self._decode([items[i] for i in dec], q_dec, stream, dec_host,
                             [dv[j] for j in i_dec], chunk=chunk)
            for i in pre:
                r, s, n, _ = items[i]
                self._prefill(r, s, n, q[offs[i]:offs[i] + n], stream, pf_host[i], dv[i_pf[i]])
            self.stats["decode_tokens"] += len(dec)
            self.stats["prefill_tokens"] += int(sum(it[2] for it in items if not it[3]))
        done = L.pa_sched_commit(self.sched, self.max_running)
        self.stats["steps"] += 1
        self.stats["finished"] += len(done)
        return done

    def _decode_host(self, items):
        """Host arrays of a decode batch: tables, lengths, work list, and the
        table width and longest length."""
        ids = [r for r, _, _, _ in items]
        # each request's length after this step is known from its item
        max_blocks = max(-(-(s + 1) // L.BLOCK_SIZE) for _, s, _, _ in items)
        tab, ln = L.pa_block_tables(self.cache.pool, ids, max_blocks)
        assert [int(x) for x in ln] == [s + 1 for _, s, _, _ in items]
        work = L.pa_decode_work_items(ln, self.partition)
        return tab, ln, work, max_blocks, int(ln.max())

    def _prefill_host(self, r: int, s: int, n: int):
        """Host table of a prefill chunk and its width."""
        max_blocks = -(-(s + n) // L.BLOCK_SIZE)
        tab, ln = L.pa_block_tables(self.cache.pool, [r], max_blocks)
        assert int(ln[0]) == s + n
        return tab[0], max_blocks

    def _decode(self, items, q: torch.Tensor, stream, host, dev, chunk=None):
        """Decode attention for the items (host: _decode_host's arrays, dev:
        device copies of its tables, lengths and work list); with chunk =
        (request, start, length, query rows, prefill host data, prefill
        device table) that prefill chunk runs in the same launch."""
        _, _, work, max_blocks, max_len = host
        d_tab, d_len, d_work = dev
        n_dec = len(items)
        ws_bytes = L.pa_decode_workspace_bytes(n_dec, self.n_q, self.d, max_len, self.partition)
        ws = self._workspace("_ws", max(ws_bytes, 16))
        out = torch.empty((n_dec, self.n_q, self.d), dtype=torch.float16, device=self.dev)
        flags = L.PA_DECODE_KEEP_KV if self.cache.shares_blocks() else 0
        # a contiguous copy of the queries (a slice of the step's fused rows
        # is not): bound to a name so it outlives every launch that reads it
        q_c = q.contiguous()
        if chunk is None:
            self.cache.decode(out, q_c, d_tab, max_blocks, d_len, n_dec, self.n_q,
                              self.scale, self.partition, max_len, d_work, len(work), ws,
                              ws_bytes, stream, flags=flags)
            self._hold(stream, q_c, out, ws)
        else:
            r, s, n, qc, (_, pf_blocks), d_ptab = chunk
            qc = qc.contiguous()
            pout = torch.empty((n, self.n_q, self.d), dtype=torch.float16, device=self.dev)
            c_dec = L.decode_batch(out, q_c, d_tab, max_blocks, d_len, n_dec,
                                   self.partition, max_len, d_work, len(work))
            c_pf = L.prefill_chunk(pout, qc, d_ptab, pf_blocks, s, n)
            mws_bytes = L.pa_mixed_workspace_bytes(c_dec, c_pf, self.n_q, self.d)
            mws = self._workspace("_ws", max(mws_bytes, 16))
            L.pa_paged_attention_mixed(c_dec, c_pf, self.cache.kv, self.n_q, self.scale, mws,
                                       mws_bytes, stream, flags=flags)
            self._hold(stream, q_c, out, qc, pout, mws)
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

    def _prefill(self, r: int, s: int, n: int, q: torch.Tensor, stream, host, d_tab):
        _, max_blocks = host
        ws_bytes = L.pa_prefill_workspace_bytes(n, self.n_q, self.d, s)
        ws = self._workspace("_pws", max(ws_bytes, 16))
        out = torch.empty((n, self.n_q, self.d), dtype=torch.float16, device=self.dev)
        q_c = q.contiguous()
        L.pa_paged_attention_prefill(out, q_c, self.cache.kv, d_tab, max_blocks, s, n,
                                     self.n_q, self.scale, ws, ws_bytes, stream)
        self._hold(stream, q_c, out, ws)
        if self.keep:
            kept = out.clone()
            for j in range(n):
                self.outputs[(r, s + j)] = (kept[j], "prefill")

    def request(self, req_id: int):
        """(computed input tokens, generated tokens, preemptions)."""
        return L.pa_sched_request(self.sched, req_id)

    def sched_stats(self) -> dict:
        return L.pa_sched_get_stats(self.sched)
