"""Run a synthetic workload's block-manager program and step on the oracle
models.  TEST INFRASTRUCTURE ONLY.

A workload (see ``synth.workloads``) is a list of add / append / fork
operations plus the K/V rows its appends store; the step then appends each
decode request's new token (and, in the mixed configuration, a prefill chunk)
before attention runs.  The order within a step follows the scheduler sketch
in ta-paperlens (blocks are reserved for every running request, then one
forward pass runs; prefill and decode may share it): reserve slots, perform the
copy-on-write copies, store the new K/V, then attend.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Tuple

import numpy as np

from .allocator import BlockPoolModel
from .attention import decode_attention_one, prefill_chunk_attention
from .pool import Fp8PoolModel, PoolModel


@dataclass
class OracleState:
    alloc: BlockPoolModel
    pool: PoolModel
    setup_slots: np.ndarray
    step_slots: np.ndarray = None
    step_copies: List[Tuple[int, int, int]] = None


def run_setup(w, bulk: bool = True, kv_dtype: str = "fp16", k_scale: float = 1.0,
              v_scale: float = 1.0) -> OracleState:
    """``kv_dtype="fp8"`` stores E4M3 codes under the given per-pool scales
    (the FP8 KV-cache variant); attention then sees the values they stand for."""
    alloc = BlockPoolModel(w.num_blocks, 16, w.free_order)
    if kv_dtype == "fp8":
        pool = Fp8PoolModel(w.num_blocks, w.n_kv, w.d, k_scale, v_scale)
    elif kv_dtype == "fp16":
        pool = PoolModel(w.num_blocks, w.n_kv, w.d)
    else:
        raise ValueError(kv_dtype)
    cursor = 0
    all_slots: List[int] = []
    for op in w.setup:
        kind = op[0]
        if kind == "add":
            alloc.add(int(op[1]))
        elif kind == "fork":
            alloc.fork(int(op[1]), int(op[2]))
        elif kind == "append":
            slots, copies = alloc.append(op[1], op[2])
            pool.copy(copies)
            n = len(slots)
            rows_k = w.setup_k[cursor:cursor + n]
            rows_v = w.setup_v[cursor:cursor + n]
            if bulk:
                pool.write_bulk(rows_k, rows_v, slots)
            else:
                pool.write(rows_k, rows_v, slots)
            cursor += n
            all_slots.extend(slots)
        else:
            raise ValueError(kind)
    assert cursor == len(w.setup_k)
    return OracleState(alloc, pool, np.asarray(all_slots, dtype=np.int64))


def run_step(w, st: OracleState) -> OracleState:
    slots, copies = st.alloc.append(w.step_ids.tolist(), w.step_n_new.tolist())
    st.pool.copy(copies)
    st.pool.write(w.step_k, w.step_v, slots)
    st.step_slots = np.asarray(slots, dtype=np.int64)
    st.step_copies = list(copies)
    return st


def decode_reference(w, st: OracleState, seq_index=None) -> np.ndarray:
    """fp64 decode outputs [B][n_q][d] (or for the listed batch indices)."""
    idx = range(w.batch) if seq_index is None else seq_index
    outs = []
    for i in idx:
        sid = int(w.decode_ids[i])
        k, v = st.pool.gather_values(st.alloc.tables[sid], st.alloc.lens[sid])
        outs.append(decode_attention_one(w.q[i], k, v, w.scale))
    return np.stack(outs)


def prefill_reference(w, st: OracleState, rows=None, heads=None) -> np.ndarray:
    pf = w.prefill
    sid = pf.seq_id
    k, v = st.pool.gather_values(st.alloc.tables[sid], st.alloc.lens[sid])
    return prefill_chunk_attention(pf.q, k, v, pf.q_start, w.scale, rows=rows, heads=heads)
