"""A paged K/V cache on one GPU, driven through the C ABI.

``PagedKVCache`` owns a host block pool (``pa_pool_*``) and the two device
pool tensors of one layer, and strings the library's calls together in the
order one step needs them (the scheduler sketch of ta-paperlens: reserve
blocks for every running request, then run the forward pass):

    pa_append_slots -> H2D(slot_mapping, copies) -> pa_copy_blocks
        -> pa_reshape_and_cache -> pa_block_tables -> H2D(tables, lens)
        -> pa_paged_attention_decode / pa_paged_attention_prefill

PyTorch only provides device memory, streams and host<->device copies; every
computation is one of the library's kernels.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np
import torch

from . import _lib as L

DEFAULT_PARTITION = 512


class PagedKVCache:
    """``kv_dtype`` "fp16" (default) or "fp8": E4M3 codes with one scale per
    pool (``k_scale``, ``v_scale``), half the bytes per token; fp16 rows are
    quantised as they are stored."""

    def __init__(self, num_blocks: int, num_kv_heads: int, head_dim: int,
                 free_order: Optional[Sequence[int]] = None, device="cuda:0",
                 fill_byte: Optional[int] = None, kv_dtype: str = "fp16",
                 k_scale: float = 1.0, v_scale: float = 1.0):
        if kv_dtype not in ("fp16", "fp8"):
            raise ValueError(f"kv_dtype must be 'fp16' or 'fp8', not {kv_dtype!r}")
        self.num_blocks = int(num_blocks)
        self.n_kv = int(num_kv_heads)
        self.d = int(head_dim)
        self.device = torch.device(device)
        self.kv_dtype = kv_dtype
        self.fp8 = kv_dtype == "fp8"
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.pool = L.pa_pool_create(self.num_blocks, free_order)
        # [block][kv head][tile of 16 slots x d values, in the library's operand order]
        shape = (self.num_blocks, self.n_kv, L.BLOCK_SIZE * self.d)
        dt = torch.uint8 if self.fp8 else torch.float16
        self.k_pool = torch.empty(shape, dtype=dt, device=self.device)
        self.v_pool = torch.empty(shape, dtype=dt, device=self.device)
        if fill_byte is not None:
            self.k_pool.view(torch.uint8).fill_(fill_byte)
            self.v_pool.view(torch.uint8).fill_(fill_byte)
        if self.fp8:
            self.kv = L.kv_view_fp8(self.k_pool, self.v_pool, self.num_blocks, self.n_kv, self.d,
                                    self.k_scale, self.v_scale)
        else:
            self.kv = L.kv_view(self.k_pool, self.v_pool, self.num_blocks, self.n_kv, self.d)

    def close(self):
        if self.pool:
            L.pa_pool_destroy(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def shares_blocks(self) -> bool:
        """True while some block is referenced by more than one sequence:
        decode then keeps K/V tiles in cache (PA_DECODE_KEEP_KV) so that a
        shared prefix is read from HBM once per kv head."""
        return L.pa_pool_get_stats(self.pool)["num_shared"] > 0

    # -- host-side request bookkeeping -------------------------------------
    def add(self, seq_id: int):
        L.pa_seq_add(self.pool, seq_id)

    def fork(self, parent: int, child: int):
        L.pa_seq_fork(self.pool, parent, child)

    def free(self, seq_id: int):
        L.pa_seq_free(self.pool, seq_id)

    def seq_len(self, seq_id: int) -> int:
        return L.pa_seq_table(self.pool, seq_id)[1]

    # -- device calls of this pool's type ------------------------------------
    def store(self, k_rows, v_rows, d_slots, n: int, stream) -> None:
        """pa_reshape_and_cache (fp16 pools) or pa_reshape_and_cache_fp8."""
        fn = L.pa_reshape_and_cache_fp8 if self.fp8 else L.pa_reshape_and_cache
        fn(k_rows, v_rows, d_slots, n, self.kv, stream)

    def copy_blocks(self, d_copies, n: int, stream) -> None:
        """pa_copy_blocks (fp16 pools) or pa_copy_blocks_fp8."""
        fn = L.pa_copy_blocks_fp8 if self.fp8 else L.pa_copy_blocks
        fn(d_copies, n, self.kv, stream)

    def decode(self, out, q, tables, max_blocks, lens, batch, n_q, scale, partition, max_len,
               items, n_items, workspace, ws_bytes, stream, flags=0) -> None:
        """pa_paged_attention_decode (fp16 pools) or pa_paged_attention_decode_fp8."""
        fn = L.pa_paged_attention_decode_fp8 if self.fp8 else L.pa_paged_attention_decode
        fn(out, q, self.kv, tables, max_blocks, lens, batch, n_q, scale, partition, max_len,
           items, n_items, workspace, ws_bytes, stream, flags=flags)

    # -- preemption by swapping ----------------------------------------------
    def gather_to_host(self, blocks, stream=None):
        """K and V tiles of `blocks` (host int32, logical order) into pinned
        host tensors [n][n_kv][16*d]: pa_gather_blocks into a device staging
        buffer, then one copy each, enqueued on `stream` (complete once the
        stream gets there)."""
        stream = stream or torch.cuda.current_stream(self.device)
        n = len(blocks)
        tile = (n, self.n_kv, L.BLOCK_SIZE * self.d)
        dt = self.k_pool.dtype
        k_host = torch.empty(tile, dtype=dt, pin_memory=True)
        v_host = torch.empty(tile, dtype=dt, pin_memory=True)
        if n:
            with torch.cuda.stream(stream):
                d_blocks = torch.from_numpy(np.ascontiguousarray(blocks, dtype=np.int32)) \
                    .pin_memory().to(self.device, non_blocking=True)
                k_buf = torch.empty(tile, dtype=dt, device=self.device)
                v_buf = torch.empty(tile, dtype=dt, device=self.device)
                L.pa_gather_blocks(d_blocks, n, self.kv, k_buf, v_buf, stream)
                k_host.copy_(k_buf, non_blocking=True)
                v_host.copy_(v_buf, non_blocking=True)
        return k_host, v_host

    def scatter_from_host(self, blocks, k_host, v_host, stream=None) -> None:
        """Write tiles saved by gather_to_host into `blocks` (pa_scatter_blocks)."""
        stream = stream or torch.cuda.current_stream(self.device)
        n = len(blocks)
        if n:
            with torch.cuda.stream(stream):
                d_blocks = torch.from_numpy(np.ascontiguousarray(blocks, dtype=np.int32)) \
                    .pin_memory().to(self.device, non_blocking=True)
                k_buf = k_host.to(self.device, non_blocking=True)
                v_buf = v_host.to(self.device, non_blocking=True)
                L.pa_scatter_blocks(d_blocks, n, self.kv, k_buf, v_buf, stream)

    def swap_out(self, seq_id: int, stream=None) -> dict:
        """Move a sequence's K/V to pinned host memory and release it
        (pa_seq_swap_out, then gather_to_host, enqueued before anything can
        reuse the blocks).  Returns what swap_in needs; the host copy is
        complete once the stream reaches the returned event."""
        stream = stream or torch.cuda.current_stream(self.device)
        blocks, length = L.pa_seq_swap_out(self.pool, seq_id)
        k_host, v_host = self.gather_to_host(blocks, stream)
        ev = torch.cuda.Event()
        ev.record(stream)
        return {"len": length, "n": len(blocks), "k": k_host, "v": v_host, "event": ev}

    def swap_in(self, seq_id: int, saved: dict, stream=None) -> np.ndarray:
        """Re-create a swapped-out sequence in fresh blocks (pa_seq_swap_in)
        and copy its K/V back.  Raises OutOfBlocksError, changing nothing,
        when the pool cannot hold it.  Returns its new blocks."""
        blocks = L.pa_seq_swap_in(self.pool, seq_id, saved["len"])
        self.scatter_from_host(blocks, saved["k"], saved["v"], stream)
        return blocks

    # -- one append: reserve, copy-on-write, store --------------------------
    def append(self, seq_ids, n_new, k_rows: torch.Tensor, v_rows: torch.Tensor,
               stream: Optional[torch.cuda.Stream] = None):
        """Reserve slots for the tokens, then store their K/V rows
        ([T][n_kv][d] fp16 on the device, in (sequence, position) order).
        Returns (slot_mapping, copies) as host arrays."""
        slots, copies = L.pa_append_slots(self.pool, seq_ids, n_new)
        T = len(slots)
        if T != k_rows.shape[0] or T != v_rows.shape[0]:
            raise ValueError(f"{T} slots reserved but {k_rows.shape[0]} K rows given")
        stream = stream or torch.cuda.current_stream(self.device)
        with torch.cuda.stream(stream):
            if len(copies):
                d_copies = torch.from_numpy(np.ascontiguousarray(copies)).to(
                    self.device, non_blocking=False)
                self.copy_blocks(d_copies, len(copies), stream)
            if T:
                d_slots = torch.from_numpy(slots).to(self.device, non_blocking=False)
                self.store(k_rows, v_rows, d_slots, T, stream)
        return slots, copies

    def tables(self, seq_ids, max_blocks: Optional[int] = None):
        """Device block tables [B][max_blocks] and lengths [B], plus the max length."""
        tab, ln, max_blocks = self.host_tables(seq_ids, max_blocks)
        return (torch.from_numpy(tab).to(self.device), torch.from_numpy(ln).to(self.device),
                int(ln.max()) if len(ln) else 0, max_blocks)

    def host_tables(self, seq_ids, max_blocks: Optional[int] = None):
        """Host block tables [B][max_blocks], lengths [B] and max_blocks."""
        seq_ids = list(seq_ids)
        if max_blocks is None:
            lens = [self.seq_len(s) for s in seq_ids]
            max_blocks = max([1] + [-(-x // L.BLOCK_SIZE) for x in lens])
        tab, ln = L.pa_block_tables(self.pool, seq_ids, max_blocks)
        return tab, ln, max_blocks


class DecodePlan:
    """Device-resident arguments of one decode launch (tables, lengths, work
    list, workspace), so repeated launches time only the kernels.
    ``worklist`` selects the work-list (persistent) form; otherwise one
    workgroup per (kv head, request, partition)."""

    def __init__(self, cache: PagedKVCache, seq_ids, num_q_heads: int, scale: float,
                 partition: int = DEFAULT_PARTITION, out: Optional[torch.Tensor] = None,
                 worklist: bool = True, keep_kv: Optional[bool] = None):
        self.cache = cache
        keep = cache.shares_blocks() if keep_kv is None else bool(keep_kv)
        self.flags = L.PA_DECODE_KEEP_KV if keep else 0
        tab, ln, self.max_blocks = cache.host_tables(seq_ids)
        self.tables = torch.from_numpy(tab).to(cache.device)
        self.lens = torch.from_numpy(ln).to(cache.device)
        self.max_len = int(ln.max()) if len(ln) else 0
        self.batch = len(ln)
        self.n_q = int(num_q_heads)
        self.scale = float(scale)
        self.partition = int(partition)
        if worklist:
            items = L.pa_decode_work_items(ln, self.partition)
            self.items = torch.from_numpy(np.ascontiguousarray(items)).to(cache.device)
            self.n_items = len(items)
        else:
            self.items, self.n_items = None, 0
        ws = L.pa_decode_workspace_bytes(self.batch, self.n_q, cache.d, self.max_len,
                                         self.partition)
        self.ws_bytes = ws
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=cache.device)
        self.out = out if out is not None else torch.empty(
            (self.batch, self.n_q, cache.d), dtype=torch.float16, device=cache.device)

    def run(self, q: torch.Tensor, stream=None) -> torch.Tensor:
        self.cache.decode(self.out, q, self.tables, self.max_blocks, self.lens, self.batch,
                          self.n_q, self.scale, self.partition, self.max_len, self.items,
                          self.n_items, self.workspace, self.ws_bytes,
                          stream or torch.cuda.current_stream(self.cache.device),
                          flags=self.flags)
        return self.out


class PrefillPlan:
    """Device-resident arguments of one prefill-chunk launch."""

    def __init__(self, cache: PagedKVCache, seq_id: int, q_start: int, chunk_len: int,
                 num_q_heads: int, scale: float):
        self.cache = cache
        tab, _, self.seq_len, self.table_len = cache.tables([seq_id])
        self.table = tab[0].contiguous()
        self.q_start, self.chunk_len = int(q_start), int(chunk_len)
        self.n_q, self.scale = int(num_q_heads), float(scale)
        ws = L.pa_prefill_workspace_bytes(self.chunk_len, self.n_q, cache.d, self.q_start)
        self.ws_bytes = ws
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=cache.device)
        self.out = torch.empty((self.chunk_len, self.n_q, cache.d), dtype=torch.float16,
                               device=cache.device)

    def run(self, q: torch.Tensor, stream=None) -> torch.Tensor:
        L.pa_paged_attention_prefill(self.out, q, self.cache.kv, self.table, self.table_len,
                                     self.q_start, self.chunk_len, self.n_q, self.scale,
                                     self.workspace, self.ws_bytes,
                                     stream or torch.cuda.current_stream(self.cache.device))
        return self.out


class MixedPlan:
    """Device-resident arguments of one mixed launch: a decode batch (work-list
    form) and one prefill chunk over the same pool (fp16 or FP8), attended by
    ``pa_paged_attention_mixed`` (``pa_paged_attention_mixed_fp8``)."""

    def __init__(self, cache: PagedKVCache, seq_ids, prefill_seq_id: int, q_start: int,
                 chunk_len: int, num_q_heads: int, scale: float,
                 partition: int = DEFAULT_PARTITION, keep_kv: Optional[bool] = None):
        self.cache = cache
        self.dec = DecodePlan(cache, seq_ids, num_q_heads, scale, partition, keep_kv=keep_kv)
        self.pf = PrefillPlan(cache, prefill_seq_id, q_start, chunk_len, num_q_heads, scale)
        self.n_q, self.scale = int(num_q_heads), float(scale)
        self.q_dec: Optional[torch.Tensor] = None
        self.q_pf: Optional[torch.Tensor] = None
        self._bind()

    def _bind(self):
        d, p = self.dec, self.pf
        self.c_dec = L.decode_batch(d.out, self.q_dec, d.tables, d.max_blocks, d.lens, d.batch,
                                    d.partition, d.max_len, d.items, d.n_items)
        self.c_pf = L.prefill_chunk(p.out, self.q_pf, p.table, p.table_len, p.q_start,
                                    p.chunk_len)
        self.ws_bytes = L.pa_mixed_workspace_bytes(self.c_dec, self.c_pf, self.n_q, self.cache.d)
        if not hasattr(self, "workspace") or self.workspace.numel() < max(self.ws_bytes, 16):
            self.workspace = torch.zeros(max(self.ws_bytes, 16), dtype=torch.uint8,
                                         device=self.cache.device)

    def run(self, q_decode: torch.Tensor, q_prefill: torch.Tensor, stream=None):
        """Returns (decode output [B][n_q][D], prefill output [C][n_q][D])."""
        if q_decode is not self.q_dec or q_prefill is not self.q_pf:
            self.q_dec, self.q_pf = q_decode, q_prefill
            self._bind()
        L.pa_paged_attention_mixed(self.c_dec, self.c_pf, self.cache.kv, self.n_q, self.scale,
                                   self.workspace, self.ws_bytes,
                                   stream or torch.cuda.current_stream(self.cache.device),
                                   flags=self.dec.flags)
        return self.dec.out, self.pf.out


def run_program(cache: PagedKVCache, setup, k_rows: torch.Tensor, v_rows: torch.Tensor):
    """Apply a list of ("add", id) / ("fork", parent, child) /
    ("append", ids, n_new) operations, taking appended rows in order."""
    cursor = 0
    for op in setup:
        if op[0] == "add":
            cache.add(int(op[1]))
        elif op[0] == "fork":
            cache.fork(int(op[1]), int(op[2]))
        elif op[0] == "append":
            n = int(sum(op[2]))
            cache.append(op[1], op[2], k_rows[cursor:cursor + n], v_rows[cursor:cursor + n])
            cursor += n
        else:
            raise ValueError(op[0])
    return cursor


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
