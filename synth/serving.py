"""Synthetic token rows and request traces for serving runs.

A serving run needs a K, V and query row for every (request, position) it
computes, and a run that preempts and recomputes a request must get the same
rows again.  So rows are a pure function of (request, position, tensor,
element): a counter-based integer hash (multiply / xor-shift steps on
31-bit values in int64, no overflow), mapped to multiples of 1/1024 in
[-1, 1), which fp16 holds exactly.  The same code runs on numpy arrays
(host) and torch tensors (device) and gives the same values.

Nothing here is attention or allocation arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

_M31 = 0x7FFFFFFF
TAG_K, TAG_V, TAG_Q = 0, 1, 2


def _mix31(h):
    h = h ^ (h >> 15)
    h = (h * 0x2C1B3C6D) & _M31
    h = h ^ (h >> 12)
    h = (h * 0x297A2D39) & _M31
    return h ^ (h >> 15)


def token_rows(req, pos, tag: int, width: int, xp=np):
    """Rows [len(req), width] for tokens (req[i], pos[i]); xp is numpy or torch
    (req, pos int64 arrays / tensors on the wanted device).  float16."""
    if xp is np:
        req = np.asarray(req, dtype=np.int64)
        pos = np.asarray(pos, dtype=np.int64)
        e = np.arange(width, dtype=np.int64)[None, :]
    else:
        e = xp.arange(width, dtype=xp.int64, device=req.device)[None, :]
    key = ((req * 131071 + pos) * 4 + tag) & _M31
    h = ((key[:, None] * 0x9E3779B1) + e * 0x85EBCA77) & _M31
    h = _mix31(_mix31(h))
    vals = (h >> 20) - 1024                      # integers in [-1024, 1023]
    if xp is np:
        return (vals.astype(np.float64) / 1024.0).astype(np.float16)
    return (vals.to(xp.float32) / 1024.0).to(xp.float16)


_KVQ_COLS = {}


def token_rows_kvq(req, pos, width_kv: int, width_q: int, xp):
    """The K, V and query rows of token_rows (tags TAG_K, TAG_V, TAG_Q) from
    one pass over [len(req), 2 * width_kv + width_q] elements: the same
    values, a third of the device launches.  xp is torch; returns three
    float16 views [len(req), width]."""
    dev = req.device
    ck = (width_kv, width_q, str(dev))
    if ck not in _KVQ_COLS:
        tag = xp.cat([xp.full((width_kv,), TAG_K, dtype=xp.int64),
                      xp.full((width_kv,), TAG_V, dtype=xp.int64),
                      xp.full((width_q,), TAG_Q, dtype=xp.int64)]).to(dev)
        e = xp.cat([xp.arange(width_kv, dtype=xp.int64), xp.arange(width_kv, dtype=xp.int64),
                    xp.arange(width_q, dtype=xp.int64)]).to(dev)
        _KVQ_COLS[ck] = (tag[None, :], (e * 0x85EBCA77)[None, :])
    tag, e_mul = _KVQ_COLS[ck]
    key = (((req * 131071 + pos) * 4)[:, None] + tag) & _M31
    h = ((key * 0x9E3779B1) + e_mul) & _M31
    h = _mix31(_mix31(h))
    rows = ((h >> 20) - 1024).to(xp.float32).div_(1024.0).to(xp.float16)
    return rows[:, :width_kv], rows[:, width_kv:2 * width_kv], rows[:, 2 * width_kv:]


@dataclass
class ServingTrace:
    """Requests (id, prompt length, output length) and the step each arrives."""
    prompt: List[int]
    output: List[int]
    arrival: List[int]


def make_trace(n: int, seed: int, prompt_median: float = 1000.0, prompt_max: int = 4096,
               out_lo: int = 64, out_hi: int = 256, arrive_over: int = 0) -> ServingTrace:
    """n requests: prompt lengths lognormal(median, sigma 1) rounded and
    clipped to [16, prompt_max], outputs uniform in [out_lo, out_hi], arrival
    steps uniform in [0, arrive_over] (sorted)."""
    rng = np.random.default_rng(seed)
    prompt = np.clip(np.rint(rng.lognormal(np.log(prompt_median), 1.0, size=n)), 16, prompt_max)
    output = rng.integers(out_lo, out_hi + 1, size=n)
    arrival = np.sort(rng.integers(0, arrive_over + 1, size=n))
    return ServingTrace([int(x) for x in prompt], [int(x) for x in output],
                        [int(x) for x in arrival])
