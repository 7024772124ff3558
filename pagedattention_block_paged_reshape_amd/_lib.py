"""ctypes binding of ``libpagedattn.so`` (argument marshalling only).

Every function here has the name of the C entry point it wraps (see
include/pa.h) and does nothing but convert arguments: Python ints, numpy
arrays for host buffers, and objects exposing ``data_ptr()`` (torch tensors)
for device buffers.  All computation happens in the library; if the library
is missing the import fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
PA_DECODE_KEEP_KV = 1  # pa_paged_attention_decode flag: K/V tiles shared between requests
PA_DECODE_SCRATCH_BYTES = 64 << 20  # partials pa_paged_attention_decode_noalloc can hold
# PA_LIBRARY selects another build of the same library (the sanitizer build
# the CPU tests can run against); by default the in-tree libpagedattn.so
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpagedattn.so")

PA_OK = 0
PA_ERR_INVALID = 1
PA_ERR_OUT_OF_BLOCKS = 2
PA_ERR_UNKNOWN_SEQ = 3
PA_ERR_EXISTS = 4
PA_ERR_CAPACITY = 5
PA_ERR_HIP = 6
PA_ERR_INTERNAL = 7
BLOCK_SIZE = 16


class PaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class OutOfBlocksError(PaError):
    pass


class pa_pool_desc(C.Structure):
    _fields_ = [("num_blocks", C.c_int32), ("block_size", C.c_int32),
                ("free_order", C.POINTER(C.c_int32))]


class pa_copy(C.Structure):
    _fields_ = [("src", C.c_int32), ("dst", C.c_int32), ("n_slots", C.c_int32)]


class pa_sched_item(C.Structure):
    _fields_ = [("req_id", C.c_int64), ("start", C.c_int32), ("n_tokens", C.c_int32),
                ("decode", C.c_int32), ("reserved", C.c_int32)]


class pa_sched_stats(C.Structure):
    _fields_ = [("n_waiting", C.c_int32), ("n_running", C.c_int32), ("steps", C.c_int64),
                ("preemptions", C.c_int64), ("finished", C.c_int64), ("n_swapped", C.c_int32),
                ("reserved", C.c_int32)]


class pa_sched_swap(C.Structure):
    _fields_ = [("req_id", C.c_int64), ("kind", C.c_int32), ("seq_len", C.c_int32),
                ("first", C.c_int64), ("n_blocks", C.c_int32), ("reserved", C.c_int32)]


class pa_pool_stats(C.Structure):
    _fields_ = [("num_blocks", C.c_int32), ("num_free", C.c_int32), ("num_seqs", C.c_int32),
                ("num_shared", C.c_int32), ("allocs", C.c_int64), ("frees", C.c_int64),
                ("cows", C.c_int64), ("num_evictable", C.c_int32), ("num_cached", C.c_int32)]


class pa_kv_view(C.Structure):
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("num_blocks", C.c_int32),
                ("block_size", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32)]


class pa_kv_view_fp8(C.Structure):
    _fields_ = [("k_pool", C.c_void_p), ("v_pool", C.c_void_p), ("num_blocks", C.c_int32),
                ("block_size", C.c_int32), ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("k_scale", C.c_float), ("v_scale", C.c_float)]


class pa_decode_batch(C.Structure):
    _fields_ = [("out", C.c_void_p), ("q", C.c_void_p), ("tables", C.c_void_p),
                ("max_blocks", C.c_int32), ("seq_lens", C.c_void_p), ("batch", C.c_int32),
                ("partition_size", C.c_int32), ("max_seq_len", C.c_int32),
                ("work_items", C.c_void_p), ("n_items", C.c_int32)]


class pa_prefill_chunk(C.Structure):
    _fields_ = [("out", C.c_void_p), ("q", C.c_void_p), ("table", C.c_void_p),
                ("table_len", C.c_int32), ("q_start", C.c_int32), ("chunk_len", C.c_int32)]


# name -> (restype, argtypes)
_P = C.c_void_p
_I32 = C.c_int32
_I64 = C.c_int64
_U64 = C.c_uint64
_SIGS = {
    "pa_status_string": (C.c_char_p, [C.c_int]),
    "pa_pool_create": (C.c_int, [C.POINTER(pa_pool_desc), C.POINTER(_P)]),
    "pa_pool_destroy": (None, [_P]),
    "pa_seq_add": (C.c_int, [_P, _I64]),
    "pa_seq_fork": (C.c_int, [_P, _I64, _I64]),
    "pa_seq_free": (C.c_int, [_P, _I64]),
    "pa_can_append": (C.c_int, [_P, _I32, _P, _P, C.POINTER(_I32)]),
    "pa_append_slots": (C.c_int, [_P, _I32, _P, _P, _P, _I64, _P, _I32, C.POINTER(_I32)]),
    "pa_block_tables": (C.c_int, [_P, _I32, _P, _I32, _P, _P]),
    "pa_seq_table": (C.c_int, [_P, _I64, _P, _I32, C.POINTER(_I32), C.POINTER(_I32)]),
    "pa_num_free_blocks": (_I32, [_P]),
    "pa_ref_count": (C.c_int, [_P, _I32, C.POINTER(_I32)]),
    "pa_pool_get_stats": (C.c_int, [_P, C.POINTER(pa_pool_stats)]),
    "pa_free_list": (C.c_int, [_P, _P, _I32, C.POINTER(_I32)]),
    "pa_evictable_list": (C.c_int, [_P, _P, _I32, C.POINTER(_I32)]),
    "pa_seq_add_cached": (C.c_int, [_P, _I64, _P, _I32, C.POINTER(_I32)]),
    "pa_seq_register": (C.c_int, [_P, _I64, _P, _I32, C.POINTER(_I32)]),
    "pa_sched_create": (C.c_int, [_P, _I32, _I32, C.POINTER(_P)]),
    "pa_sched_destroy": (None, [_P]),
    "pa_sched_add_request": (C.c_int, [_P, _I64, _I32, _I32]),
    "pa_sched_schedule": (C.c_int, [_P, _P, _I32, C.POINTER(_I32), _P, C.c_int64, _P, _I32,
                                    C.POINTER(_I32), _P, _I32, C.POINTER(_I32)]),
    "pa_sched_set_swap": (C.c_int, [_P, _I32]),
    "pa_sched_swaps": (C.c_int, [_P, _P, _I32, C.POINTER(_I32), _P, _I64, C.POINTER(_I64)]),
    "pa_sched_commit": (C.c_int, [_P, _P, _I32, C.POINTER(_I32)]),
    "pa_sched_get_stats": (C.c_int, [_P, C.POINTER(pa_sched_stats)]),
    "pa_sched_request": (C.c_int, [_P, _I64, C.POINTER(_I32), C.POINTER(_I32), C.POINTER(_I32)]),
    "pa_pool_check": (C.c_int, [_P]),
    "pa_kv_bytes_per_token": (_U64, [_I32, _I32, _I32, _I32]),
    "pa_reshape_and_cache": (C.c_int, [_P, _P, _P, _I32, pa_kv_view, _P]),
    "pa_copy_blocks": (C.c_int, [_P, _I32, pa_kv_view, _P]),
    "pa_decode_workspace_bytes": (_U64, [_I32, _I32, _I32, _I32, _I32]),
    "pa_decode_work_items": (_I32, [_P, _I32, _I32, _P, _I32]),
    "pa_paged_attention_decode": (C.c_int, [_P, _P, pa_kv_view, _P, _I32, _P, _I32, _I32,
                                            C.c_float, _I32, _I32, _P, _I32, _P, _U64, C.c_uint32,
                                            _P]),
    "pa_paged_attention_decode_noalloc": (C.c_int, [_P, _P, pa_kv_view, _P, _I32, _P, _I32,
                                                    _I32, C.c_float, _I32, _I32, _P, _I32,
                                                    C.c_uint32, _P]),
    "pa_reshape_and_cache_fp8": (C.c_int, [_P, _P, _P, _I32, pa_kv_view_fp8, _P]),
    "pa_copy_blocks_fp8": (C.c_int, [_P, _I32, pa_kv_view_fp8, _P]),
    "pa_paged_attention_decode_fp8": (C.c_int, [_P, _P, pa_kv_view_fp8, _P, _I32, _P, _I32, _I32,
                                                C.c_float, _I32, _I32, _P, _I32, _P, _U64,
                                                C.c_uint32, _P]),
    "pa_prefill_workspace_bytes": (_U64, [_I32, _I32, _I32, _I32]),
    "pa_paged_attention_prefill": (C.c_int, [_P, _P, pa_kv_view, _P, _I32, _I32, _I32, _I32,
                                             C.c_float, _P, _U64, _P]),
    "pa_paged_attention_prefill_fp8": (C.c_int, [_P, _P, pa_kv_view_fp8, _P, _I32, _I32, _I32,
                                                 _I32, C.c_float, _P, _U64, _P]),
    "pa_seq_swap_out": (C.c_int, [_P, _I64, _P, _I32, C.POINTER(_I32), C.POINTER(_I32)]),
    "pa_seq_swap_in": (C.c_int, [_P, _I64, _I32, _P, _I32, C.POINTER(_I32)]),
    "pa_host_device_pointer": (C.c_int, [_P, C.POINTER(C.c_void_p)]),
    "pa_stage_copy": (C.c_int, [_P, _P, C.c_uint64, _P]),
    "pa_stage_update": (C.c_int, [_P, _P, C.c_uint64, _P, C.c_int64, _P, C.c_int64, _P]),
    "pa_gather_blocks": (C.c_int, [_P, _I32, pa_kv_view, _P, _P, _P]),
    "pa_scatter_blocks": (C.c_int, [_P, _I32, pa_kv_view, _P, _P, _P]),
    "pa_gather_blocks_fp8": (C.c_int, [_P, _I32, pa_kv_view_fp8, _P, _P, _P]),
    "pa_scatter_blocks_fp8": (C.c_int, [_P, _I32, pa_kv_view_fp8, _P, _P, _P]),
    "pa_mixed_workspace_bytes": (_U64, [C.POINTER(pa_decode_batch), C.POINTER(pa_prefill_chunk),
                                        _I32, _I32]),
    "pa_paged_attention_mixed": (C.c_int, [C.POINTER(pa_decode_batch),
                                           C.POINTER(pa_prefill_chunk), pa_kv_view, _I32,
                                           C.c_float, _P, _U64, C.c_uint32, _P]),
    "pa_paged_attention_mixed_fp8": (C.c_int, [C.POINTER(pa_decode_batch),
                                               C.POINTER(pa_prefill_chunk), pa_kv_view_fp8, _I32,
                                               C.c_float, _P, _U64, C.c_uint32, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python pagedattention_block_paged_reshape_amd/build.py` (no fallback exists)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()
EXPORTED = tuple(_SIGS)


def status_string(status: int) -> str:
    return LIB.pa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status == PA_ERR_OUT_OF_BLOCKS:
        raise OutOfBlocksError(status, where)
    if status != PA_OK:
        raise PaError(status, where)


def _host(a, dtype) -> np.ndarray:
    arr = np.ascontiguousarray(np.asarray(a, dtype=dtype))
    return arr


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data if a.size else 0


def _dptr(t) -> Optional[int]:
    """Device pointer of a torch tensor (or an int address, or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ---------------------------------------------------------------- host pool

def pa_pool_create(num_blocks: int, free_order: Optional[Sequence[int]] = None,
                   block_size: int = BLOCK_SIZE) -> int:
    order = None if free_order is None else _host(free_order, np.int32)
    desc = pa_pool_desc(int(num_blocks), int(block_size),
                        None if order is None else order.ctypes.data_as(C.POINTER(C.c_int32)))
    handle = _P()
    _check(LIB.pa_pool_create(C.byref(desc), C.byref(handle)), "pa_pool_create")
    return handle.value


def pa_pool_destroy(pool: int) -> None:
    LIB.pa_pool_destroy(pool)


def pa_seq_add(pool: int, seq_id: int) -> None:
    _check(LIB.pa_seq_add(pool, int(seq_id)), "pa_seq_add")


def pa_seq_fork(pool: int, parent: int, child: int) -> None:
    _check(LIB.pa_seq_fork(pool, int(parent), int(child)), "pa_seq_fork")


def pa_seq_add_cached(pool: int, seq_id: int, tokens) -> int:
    """New request starting with the cached blocks of ``tokens``; returns the
    number of cached tokens (its length)."""
    t = _host(tokens, np.int32)
    out = _I32()
    _check(LIB.pa_seq_add_cached(pool, int(seq_id), t.ctypes.data if len(t) else None, len(t),
                                 C.byref(out)), "pa_seq_add_cached")
    return out.value


def pa_seq_register(pool: int, seq_id: int, tokens) -> int:
    """Cache the request's full blocks within its first len(tokens) tokens;
    returns how many blocks were newly cached."""
    t = _host(tokens, np.int32)
    out = _I32()
    _check(LIB.pa_seq_register(pool, int(seq_id), t.ctypes.data if len(t) else None, len(t),
                               C.byref(out)), "pa_seq_register")
    return out.value


def pa_seq_free(pool: int, seq_id: int) -> None:
    _check(LIB.pa_seq_free(pool, int(seq_id)), "pa_seq_free")


def pa_can_append(pool: int, seq_ids, n_new) -> int:
    ids = _host(seq_ids, np.int64)
    nn = _host(n_new, np.int32)
    out = _I32()
    _check(LIB.pa_can_append(pool, len(ids), _ptr(ids), _ptr(nn), C.byref(out)), "pa_can_append")
    return out.value


def pa_append_slots(pool: int, seq_ids, n_new, slots_out: Optional[np.ndarray] = None):
    """Returns (slot_mapping int32[T], copies int32[n][3] as (src, dst, n_slots)).
    ``slots_out`` (contiguous int32, >= T entries) receives the slots in place."""
    ids = _host(seq_ids, np.int64)
    nn = _host(n_new, np.int32)
    T = int(nn.sum()) if nn.size else 0
    if slots_out is not None:
        if slots_out.dtype != np.int32 or not slots_out.flags.c_contiguous or slots_out.size < T:
            raise ValueError("slots_out must be contiguous int32 with room for every slot")
        slots = slots_out
    else:
        slots = np.empty(max(T, 1), dtype=np.int32)
    cap = len(ids)
    copies = (pa_copy * max(cap, 1))()
    n_copies = _I32()
    _check(LIB.pa_append_slots(pool, len(ids), _ptr(ids), _ptr(nn), slots.ctypes.data, T,
                               C.addressof(copies), cap, C.byref(n_copies)), "pa_append_slots")
    cp = np.array([(c.src, c.dst, c.n_slots) for c in copies[:n_copies.value]],
                  dtype=np.int32).reshape(-1, 3)
    return slots[:T], cp


def pa_block_tables(pool: int, seq_ids, max_blocks: int, tables: Optional[np.ndarray] = None,
                    lens: Optional[np.ndarray] = None):
    """Host tables [n][max_blocks] and lengths [n]; ``tables``/``lens`` may be
    caller buffers (contiguous int32) written in place."""
    ids = _host(seq_ids, np.int64)
    if tables is None:
        tables = np.empty((len(ids), max(int(max_blocks), 0)), dtype=np.int32)
    if lens is None:
        lens = np.empty(len(ids), dtype=np.int32)
    for a, need in ((tables, len(ids) * max(int(max_blocks), 0)), (lens, len(ids))):
        if a.dtype != np.int32 or not a.flags.c_contiguous or a.size < need:
            raise ValueError("tables/lens must be contiguous int32 buffers of the right size")
    _check(LIB.pa_block_tables(pool, len(ids), _ptr(ids), int(max_blocks), _ptr(tables),
                               _ptr(lens)), "pa_block_tables")
    return tables, lens


def pa_seq_table(pool: int, seq_id: int):
    nb, ln = _I32(), _I32()
    st = LIB.pa_seq_table(pool, int(seq_id), None, 0, C.byref(nb), C.byref(ln))
    if st not in (PA_OK, PA_ERR_CAPACITY):
        _check(st, "pa_seq_table")
    buf = np.empty(max(nb.value, 1), dtype=np.int32)
    _check(LIB.pa_seq_table(pool, int(seq_id), buf.ctypes.data, nb.value, C.byref(nb),
                            C.byref(ln)), "pa_seq_table")
    return buf[:nb.value], ln.value


def pa_num_free_blocks(pool: int) -> int:
    return int(LIB.pa_num_free_blocks(pool))


def pa_ref_count(pool: int, block: int) -> int:
    out = _I32()
    _check(LIB.pa_ref_count(pool, int(block), C.byref(out)), "pa_ref_count")
    return out.value


def pa_pool_get_stats(pool: int) -> dict:
    s = pa_pool_stats()
    _check(LIB.pa_pool_get_stats(pool, C.byref(s)), "pa_pool_get_stats")
    return {k: getattr(s, k) for k, _ in pa_pool_stats._fields_ if k != "reserved"}


def pa_sched_create(pool: int, token_budget: int, max_running: int) -> int:
    out = _P()
    _check(LIB.pa_sched_create(pool, int(token_budget), int(max_running), C.byref(out)),
           "pa_sched_create")
    return out.value


def pa_sched_destroy(sched: int) -> None:
    LIB.pa_sched_destroy(sched)


def pa_sched_add_request(sched: int, req_id: int, prompt_len: int, output_len: int) -> None:
    _check(LIB.pa_sched_add_request(sched, int(req_id), int(prompt_len), int(output_len)),
           "pa_sched_add_request")


def pa_sched_schedule(sched: int, token_budget: int, max_running: int) -> dict:
    """Plan one step; buffers are sized from the scheduler's own limits."""
    items = (pa_sched_item * max_running)()
    slots = np.empty(max(token_budget, 1), dtype=np.int32)
    copies = np.empty((max(max_running, 1), 3), dtype=np.int32)
    pre = np.empty(max(max_running, 1), dtype=np.int64)
    ni, nc, npre = _I32(), _I32(), _I32()
    _check(LIB.pa_sched_schedule(sched, items, max_running, C.byref(ni), slots.ctypes.data,
                                 token_budget, copies.ctypes.data, max_running, C.byref(nc),
                                 pre.ctypes.data, max_running, C.byref(npre)),
           "pa_sched_schedule")
    its = [(items[i].req_id, items[i].start, items[i].n_tokens, items[i].decode)
           for i in range(ni.value)]
    n_slots = sum(it[2] for it in its)
    return {"items": its, "slots": slots[:n_slots].copy(), "copies": copies[:nc.value].copy(),
            "preempted": pre[:npre.value].tolist()}


def pa_sched_set_swap(sched: int, enable: bool) -> None:
    _check(LIB.pa_sched_set_swap(sched, 1 if enable else 0), "pa_sched_set_swap")


def pa_sched_swaps(sched: int) -> list:
    """The planned step's transfers, in the order to run them: a list of
    (request, "out" | "in", tokens held, blocks in logical order)."""
    n, nb = _I32(), _I64()
    st = LIB.pa_sched_swaps(sched, None, 0, C.byref(n), None, 0, C.byref(nb))
    if st == PA_OK:
        return []
    if st != PA_ERR_CAPACITY:
        _check(st, "pa_sched_swaps")
    ops = (pa_sched_swap * n.value)()
    blocks = np.empty(max(nb.value, 1), dtype=np.int32)
    _check(LIB.pa_sched_swaps(sched, ops, n.value, C.byref(n), blocks.ctypes.data, nb.value,
                              C.byref(nb)), "pa_sched_swaps")
    return [(ops[i].req_id, "out" if ops[i].kind == 0 else "in", ops[i].seq_len,
             blocks[ops[i].first:ops[i].first + ops[i].n_blocks].copy()) for i in range(n.value)]


def pa_sched_commit(sched: int, cap: int) -> list:
    out = np.empty(max(cap, 1), dtype=np.int64)
    n = _I32()
    _check(LIB.pa_sched_commit(sched, out.ctypes.data, int(cap), C.byref(n)), "pa_sched_commit")
    return out[:n.value].tolist()


def pa_sched_get_stats(sched: int) -> dict:
    st = pa_sched_stats()
    _check(LIB.pa_sched_get_stats(sched, C.byref(st)), "pa_sched_get_stats")
    return {k: getattr(st, k) for k, _ in pa_sched_stats._fields_}


def pa_sched_request(sched: int, req_id: int):
    c, g, p = _I32(), _I32(), _I32()
    _check(LIB.pa_sched_request(sched, int(req_id), C.byref(c), C.byref(g), C.byref(p)),
           "pa_sched_request")
    return c.value, g.value, p.value


def pa_evictable_list(pool: int) -> np.ndarray:
    n = _I32()
    LIB.pa_evictable_list(pool, None, 0, C.byref(n))
    buf = np.empty(max(n.value, 1), dtype=np.int32)
    _check(LIB.pa_evictable_list(pool, buf.ctypes.data, n.value, C.byref(n)), "pa_evictable_list")
    return buf[:n.value]


def pa_free_list(pool: int) -> np.ndarray:
    n = _I32()
    LIB.pa_free_list(pool, None, 0, C.byref(n))
    buf = np.empty(max(n.value, 1), dtype=np.int32)
    _check(LIB.pa_free_list(pool, buf.ctypes.data, n.value, C.byref(n)), "pa_free_list")
    return buf[:n.value]


def pa_pool_check(pool: int) -> None:
    _check(LIB.pa_pool_check(pool), "pa_pool_check")


def pa_kv_bytes_per_token(layers: int, num_kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return int(LIB.pa_kv_bytes_per_token(layers, num_kv_heads, head_dim, dtype_bytes))


# ------------------------------------------------------------------ device

def kv_view(k_pool, v_pool, num_blocks: int, num_kv_heads: int, head_dim: int) -> pa_kv_view:
    return pa_kv_view(_dptr(k_pool), _dptr(v_pool), int(num_blocks), BLOCK_SIZE,
                      int(num_kv_heads), int(head_dim))


def kv_view_fp8(k_pool, v_pool, num_blocks: int, num_kv_heads: int, head_dim: int,
                k_scale: float, v_scale: float) -> pa_kv_view_fp8:
    return pa_kv_view_fp8(_dptr(k_pool), _dptr(v_pool), int(num_blocks), BLOCK_SIZE,
                          int(num_kv_heads), int(head_dim), float(k_scale), float(v_scale))


def pa_reshape_and_cache(k, v, slot_mapping, num_tokens: int, kv: pa_kv_view, stream=None) -> None:
    _check(LIB.pa_reshape_and_cache(_dptr(k), _dptr(v), _dptr(slot_mapping), int(num_tokens), kv,
                                    _stream(stream)), "pa_reshape_and_cache")


def pa_copy_blocks(copies, n: int, kv: pa_kv_view, stream=None) -> None:
    _check(LIB.pa_copy_blocks(_dptr(copies), int(n), kv, _stream(stream)), "pa_copy_blocks")


def pa_reshape_and_cache_fp8(k, v, slot_mapping, num_tokens: int, kv: pa_kv_view_fp8,
                             stream=None) -> None:
    _check(LIB.pa_reshape_and_cache_fp8(_dptr(k), _dptr(v), _dptr(slot_mapping), int(num_tokens),
                                        kv, _stream(stream)), "pa_reshape_and_cache_fp8")


def pa_copy_blocks_fp8(copies, n: int, kv: pa_kv_view_fp8, stream=None) -> None:
    _check(LIB.pa_copy_blocks_fp8(_dptr(copies), int(n), kv, _stream(stream)),
           "pa_copy_blocks_fp8")


def pa_decode_workspace_bytes(batch: int, num_q_heads: int, head_dim: int, max_seq_len: int,
                              partition_size: int) -> int:
    return int(LIB.pa_decode_workspace_bytes(batch, num_q_heads, head_dim, max_seq_len,
                                             partition_size))


def pa_decode_work_items(seq_lens, partition_size: int, out: Optional[np.ndarray] = None):
    """Host work list (int32, largest first) for the work-list decode form.
    ``out`` (contiguous int32) receives it in place when large enough."""
    lens = _host(seq_lens, np.int32)
    n = int(LIB.pa_decode_work_items(_ptr(lens), len(lens), int(partition_size), None, 0))
    if n < 0:
        _check(-n, "pa_decode_work_items")
    if out is None or out.size < n:
        out = np.empty(max(n, 1), dtype=np.int32)
    elif out.dtype != np.int32 or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous int32 array")
    m = int(LIB.pa_decode_work_items(_ptr(lens), len(lens), int(partition_size), out.ctypes.data,
                                     out.size))
    if m != n:
        raise PaError(PA_ERR_INTERNAL, "pa_decode_work_items")
    return out[:n]


def pa_paged_attention_decode(out, q, kv: pa_kv_view, tables, max_blocks: int, seq_lens,
                              batch: int, num_q_heads: int, scale: float, partition_size: int,
                              max_seq_len: int, work_items, n_items: int, workspace,
                              workspace_bytes: int, stream=None, flags: int = 0) -> None:
    _check(LIB.pa_paged_attention_decode(_dptr(out), _dptr(q), kv, _dptr(tables), int(max_blocks),
                                         _dptr(seq_lens), int(batch), int(num_q_heads),
                                         float(scale), int(partition_size), int(max_seq_len),
                                         _dptr(work_items), int(n_items), _dptr(workspace),
                                         int(workspace_bytes), int(flags), _stream(stream)),
           "pa_paged_attention_decode")


def pa_paged_attention_decode_noalloc(out, q, kv: pa_kv_view, tables, max_blocks: int, seq_lens,
                                      batch: int, num_q_heads: int, scale: float,
                                      partition_size: int, max_seq_len: int, work_items,
                                      n_items: int, stream=None, flags: int = 0) -> None:
    _check(LIB.pa_paged_attention_decode_noalloc(
        _dptr(out), _dptr(q), kv, _dptr(tables), int(max_blocks), _dptr(seq_lens), int(batch),
        int(num_q_heads), float(scale), int(partition_size), int(max_seq_len),
        _dptr(work_items), int(n_items), int(flags), _stream(stream)),
        "pa_paged_attention_decode_noalloc")


def pa_paged_attention_decode_fp8(out, q, kv: pa_kv_view_fp8, tables, max_blocks: int, seq_lens,
                                  batch: int, num_q_heads: int, scale: float, partition_size: int,
                                  max_seq_len: int, work_items, n_items: int, workspace,
                                  workspace_bytes: int, stream=None, flags: int = 0) -> None:
    _check(LIB.pa_paged_attention_decode_fp8(_dptr(out), _dptr(q), kv, _dptr(tables),
                                             int(max_blocks), _dptr(seq_lens), int(batch),
                                             int(num_q_heads), float(scale), int(partition_size),
                                             int(max_seq_len), _dptr(work_items), int(n_items),
                                             _dptr(workspace), int(workspace_bytes), int(flags),
                                             _stream(stream)), "pa_paged_attention_decode_fp8")


def pa_prefill_workspace_bytes(chunk_len: int, num_q_heads: int, head_dim: int,
                               q_start: int) -> int:
    return int(LIB.pa_prefill_workspace_bytes(chunk_len, num_q_heads, head_dim, q_start))


def pa_paged_attention_prefill(out, q, kv, table, table_len: int, q_start: int,
                               chunk_len: int, num_q_heads: int, scale: float, workspace,
                               workspace_bytes: int, stream=None) -> None:
    """fp16 pools (pa_kv_view) or FP8 pools (pa_kv_view_fp8: the _fp8 entry point)."""
    fn = LIB.pa_paged_attention_prefill_fp8 if isinstance(kv, pa_kv_view_fp8) \
        else LIB.pa_paged_attention_prefill
    _check(fn(_dptr(out), _dptr(q), kv, _dptr(table), int(table_len), int(q_start),
              int(chunk_len), int(num_q_heads), float(scale), _dptr(workspace),
              int(workspace_bytes), _stream(stream)), "pa_paged_attention_prefill")


def decode_batch(out, q, tables, max_blocks: int, seq_lens, batch: int, partition_size: int,
                 max_seq_len: int, work_items, n_items: int) -> pa_decode_batch:
    return pa_decode_batch(_dptr(out), _dptr(q), _dptr(tables), int(max_blocks), _dptr(seq_lens),
                           int(batch), int(partition_size), int(max_seq_len), _dptr(work_items),
                           int(n_items))


def prefill_chunk(out, q, table, table_len: int, q_start: int, chunk_len: int) -> pa_prefill_chunk:
    return pa_prefill_chunk(_dptr(out), _dptr(q), _dptr(table), int(table_len), int(q_start),
                            int(chunk_len))


def pa_mixed_workspace_bytes(dec: pa_decode_batch, pf: pa_prefill_chunk, num_q_heads: int,
                             head_dim: int) -> int:
    return int(LIB.pa_mixed_workspace_bytes(C.byref(dec), C.byref(pf), int(num_q_heads),
                                            int(head_dim)))


def pa_paged_attention_mixed(dec: pa_decode_batch, pf: pa_prefill_chunk, kv: pa_kv_view,
                             num_q_heads: int, scale: float, workspace, workspace_bytes: int,
                             stream=None, flags: int = 0) -> None:
    """fp16 pools (pa_kv_view) or FP8 pools (pa_kv_view_fp8: the _fp8 entry point)."""
    fn = LIB.pa_paged_attention_mixed_fp8 if isinstance(kv, pa_kv_view_fp8) \
        else LIB.pa_paged_attention_mixed
    _check(fn(C.byref(dec), C.byref(pf), kv, int(num_q_heads), float(scale), _dptr(workspace),
              int(workspace_bytes), int(flags), _stream(stream)), "pa_paged_attention_mixed")


def pa_seq_swap_out(pool: int, seq_id: int):
    """Release a sequence for swapping; returns (blocks in logical order, length)."""
    n = C.c_int32(0)
    ln = C.c_int32(0)
    st = LIB.pa_seq_swap_out(pool, int(seq_id), None, 0, C.byref(n), C.byref(ln))
    if st == PA_ERR_CAPACITY:
        # ask again with room for every block (the failed call changed nothing)
        table, _ = pa_seq_table(pool, seq_id)
        out = np.empty(max(len(table), 1), dtype=np.int32)
        st = LIB.pa_seq_swap_out(pool, int(seq_id), out.ctypes.data, out.size, C.byref(n),
                                 C.byref(ln))
        _check(st, "pa_seq_swap_out")
        return out[:n.value], ln.value
    _check(st, "pa_seq_swap_out")
    return np.empty(0, dtype=np.int32), ln.value


def pa_seq_swap_in(pool: int, seq_id: int, seq_len: int) -> np.ndarray:
    """Re-create a swapped sequence with fresh blocks; returns them in logical order."""
    n_need = -(-int(seq_len) // BLOCK_SIZE)
    out = np.empty(max(n_need, 1), dtype=np.int32)
    n = C.c_int32(0)
    _check(LIB.pa_seq_swap_in(pool, int(seq_id), int(seq_len), out.ctypes.data, out.size,
                              C.byref(n)), "pa_seq_swap_in")
    return out[:n.value]


def pa_host_device_pointer(host) -> int:
    """Device address of pinned host memory (a pin_memory tensor or an int
    host address)."""
    addr = host if isinstance(host, int) else host.data_ptr()
    out = C.c_void_p()
    _check(LIB.pa_host_device_pointer(addr, C.byref(out)), "pa_host_device_pointer")
    return int(out.value)


def pa_stage_copy(src, dst, nbytes: int, stream=None) -> None:
    _check(LIB.pa_stage_copy(_dptr(src), _dptr(dst), int(nbytes), _stream(stream)),
           "pa_stage_copy")


def pa_stage_update(src, dst, nbytes: int, updates, n_updates: int, target, target_len: int,
                    stream=None) -> None:
    _check(LIB.pa_stage_update(_dptr(src), _dptr(dst), int(nbytes), _dptr(updates),
                               int(n_updates), _dptr(target), int(target_len), _stream(stream)),
           "pa_stage_update")


def pa_gather_blocks(blocks, n: int, kv, k_out, v_out, stream=None) -> None:
    fn = LIB.pa_gather_blocks_fp8 if isinstance(kv, pa_kv_view_fp8) else LIB.pa_gather_blocks
    _check(fn(_dptr(blocks), int(n), kv, _dptr(k_out), _dptr(v_out), _stream(stream)),
           "pa_gather_blocks")


def pa_scatter_blocks(blocks, n: int, kv, k_in, v_in, stream=None) -> None:
    fn = LIB.pa_scatter_blocks_fp8 if isinstance(kv, pa_kv_view_fp8) else LIB.pa_scatter_blocks
    _check(fn(_dptr(blocks), int(n), kv, _dptr(k_in), _dptr(v_in), _stream(stream)),
           "pa_scatter_blocks")
