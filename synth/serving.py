"""Synthetic token rows and request traces for serving runs.

A serving run needs a K, V and query row for every (request, position) it
computes, and a run that preempts and recomputes a request must get the same
rows again.  So rows are a pure function of (request, position, tensor,
element): a counter-based integer hash (a 31-bit key per token and tensor,
then multiply / xor-shift steps in int32 with wrap-around products and
arithmetic shifts, which numpy and torch compute alike), mapped to multiples
of 1/1024 in [-1, 1), which fp16 holds exactly.  The same code runs on numpy arrays
(host) and torch tensors (device) and gives the same values.

Nothing here is attention or allocation arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np

_M31 = 0x7FFFFFFF
TAG_K, TAG_V, TAG_Q = 0, 1, 2
# odd multipliers below 2^31 (they fit int32 on both sides)
_C_KEY, _C_ELEM, _C_MIX1, _C_MIX2 = 0x1E3779B1, 0x05EBCA77, 0x2C1B3C6D, 0x297A2D39


def _token_key(req, pos, tag):
    """31-bit key of (request, position, tensor) in int64 (no overflow)."""
    return ((req * 131071 + pos) * 4 + tag) & _M31


def _rows_from_keys(key32, e_mul, xp):
    """key32 [T] int32 keys times _C_KEY, e_mul [W] int32 element index times
    _C_ELEM (both wrapped to int32): an int32 hash per (key, element) with
    wrap-around products and arithmetic shifts, which numpy and torch compute
    alike, mapped to multiples of 1/1024 in [-1, 1) as float16."""
    h = key32[:, None] + e_mul[None, :]
    h = h ^ (h >> 15)
    h = h * _C_MIX1
    h = h ^ (h >> 13)
    h = h * _C_MIX2
    h = h ^ (h >> 16)
    vals = ((h >> 8) & 2047) - 1024               # integers in [-1024, 1023]
    if xp is np:
        return vals.astype(np.float16) / np.float16(1024.0)
    return vals.to(xp.float16) / 1024.0


def token_rows(req, pos, tag: int, width: int, xp=np):
    """Rows [len(req), width] for tokens (req[i], pos[i]); xp is numpy or torch
    (req, pos int64 arrays / tensors on the wanted device).  float16."""
    if xp is np:
        req = np.asarray(req, dtype=np.int64)
        pos = np.asarray(pos, dtype=np.int64)
        key32 = (_token_key(req, pos, tag) * _C_KEY & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
        e_mul = (np.arange(width, dtype=np.int64) * _C_ELEM & 0xFFFFFFFF).astype(
            np.uint32).view(np.int32)
        return _rows_from_keys(key32, e_mul, np)
    key32 = _wrap32(_token_key(req, pos, tag) * _C_KEY, xp)
    e_mul = _wrap32(xp.arange(width, dtype=xp.int64, device=req.device) * _C_ELEM, xp)
    return _rows_from_keys(key32, e_mul, xp)


def _wrap32(x, xp):
    """int64 tensor -> int32 with the same low 32 bits."""
    x = x & 0xFFFFFFFF
    return (x - ((x >> 31) << 32)).to(xp.int32)


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
        _KVQ_COLS[ck] = (tag, _wrap32(e * _C_ELEM, xp))
    tag, e_mul = _KVQ_COLS[ck]
    base = (req * 131071 + pos) * 4
    # per (token, tag) keys, then each column picks its tag's key
    keys = _wrap32(((base[:, None] + xp.arange(3, device=dev)[None, :]) & _M31) * _C_KEY, xp)
    kcol = keys.index_select(1, tag)                 # [T, W] int32
    h = kcol + e_mul[None, :]
    h = h ^ (h >> 15)
    h = h * _C_MIX1
    h = h ^ (h >> 13)
    h = h * _C_MIX2
    h = h ^ (h >> 16)
    rows = (((h >> 8) & 2047) - 1024).to(xp.float16) / 1024.0
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
