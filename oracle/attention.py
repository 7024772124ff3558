"""Oracle attention and KV accounting in fp64.  TEST INFRASTRUCTURE ONLY.

Paged attention changes where the K/V bytes live, not what is computed: the
kernel follows the block table to collect K and V while computing
(ta-paperlens, "fragmentation and PagedAttention" section), and paging lets
physically scattered blocks act as one logically contiguous sequence
(media.tcdigital.jp, "logical/physical block mapping").  So the result is
ordinary scaled-dot-product softmax attention over the logically gathered
sequence, which is what this module writes out:

    s_j = scale * <q, k_j>,  p = exp(s - max s) / sum exp(s - max s),  o = sum_j p_j v_j

Grouped-query attention: query head h reads KV head floor(h / G) with
G = n_q / n_kv (contiguous groups; the pages name "GQA: 8 KV heads" in the
youngju.dev KV-size example without fixing the map).

Prefill (ta-paperlens, "prefill grows with the square of the length", FIG 1;
ngrok summary, chunked prefill): row r of a chunk that starts at absolute
position P0 attends to keys 0..P0 + r inclusive (causal).
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def _softmax_weighted_sum(s: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Two-pass softmax of the last axis of ``s`` applied to ``v``."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    p = e / np.sum(e, axis=-1, keepdims=True)
    return p @ v


def decode_attention_one(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """One request: q [n_q][d], k and v [L][n_kv][d] (logical order).
    Returns o [n_q][d] in fp64."""
    q = q.astype(np.float64)
    k = k.astype(np.float64)
    v = v.astype(np.float64)
    n_q, d = q.shape
    n_kv = k.shape[1]
    assert n_q % n_kv == 0
    G = n_q // n_kv
    out = np.empty((n_q, d), dtype=np.float64)
    for g in range(n_kv):
        kg = k[:, g, :]                    # [L][d]
        vg = v[:, g, :]
        qh = q[g * G:(g + 1) * G, :]       # [G][d]
        s = scale * (qh @ kg.T)            # [G][L]
        out[g * G:(g + 1) * G] = _softmax_weighted_sum(s, vg)
    return out


def decode_attention(q: np.ndarray, ks: Sequence[np.ndarray], vs: Sequence[np.ndarray],
                     scale: float) -> np.ndarray:
    """Batch of requests: q [B][n_q][d]; ks[i], vs[i] are request i's logical
    K and V, [L_i][n_kv][d].  Returns [B][n_q][d] fp64."""
    return np.stack([decode_attention_one(q[i], ks[i], vs[i], scale) for i in range(len(ks))])


def prefill_chunk_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_start: int,
                            scale: float, rows: Optional[Sequence[int]] = None,
                            heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Causal attention of a prefill chunk.

    q [C][n_q][d] holds the chunk's queries at absolute positions q_start + r;
    k, v [>= q_start + C][n_kv][d] are the request's logical K/V (the chunk's
    own rows included).  Row r attends keys 0..q_start + r.  ``rows`` and
    ``heads`` select a subset (for sampled checks at full size).  Returns
    [len(rows)][len(heads)][d] fp64."""
    C, n_q, d = q.shape
    n_kv = k.shape[1]
    G = n_q // n_kv
    rows = list(range(C)) if rows is None else [int(r) for r in rows]
    heads = list(range(n_q)) if heads is None else [int(h) for h in heads]
    out = np.empty((len(rows), len(heads), d), dtype=np.float64)
    r_arr = np.asarray(rows, dtype=np.int64)
    n_keys = q_start + int(r_arr.max()) + 1
    for hi, h in enumerate(heads):
        g = h // G
        kg = k[:n_keys, g, :].astype(np.float64)
        vg = v[:n_keys, g, :].astype(np.float64)
        qh = q[r_arr, h, :].astype(np.float64)             # [R][d]
        s = scale * (qh @ kg.T)                            # [R][n_keys]
        allowed = np.arange(n_keys)[None, :] <= (q_start + r_arr)[:, None]
        s = np.where(allowed, s, -np.inf)
        out[:, hi, :] = _softmax_weighted_sum(s, vg)
    return out


# -- KV accounting ----------------------------------------------------------

def kv_bytes_per_token(layers: int, n_kv: int, d: int, dtype_bytes: int) -> int:
    """Bytes of K and V one token occupies: 2 (K and V) x layers x KV heads x
    head_dim x bytes per element (ta-paperlens, KV-size example after eq. 1;
    youngju.dev, KV-cache size function)."""
    return 2 * layers * n_kv * d * dtype_bytes


def kv_cache_size_gib(layers: int, heads: int, d: int, seq_len: int, batch: int,
                      dtype_bytes: int = 2) -> float:
    """youngju.dev KV-cache size function: the per-token bytes times tokens
    times requests, in GiB (2**30 bytes)."""
    return kv_bytes_per_token(layers, heads, d, dtype_bytes) * seq_len * batch / float(1 << 30)


def contiguous_waste(used: Sequence[int], reserved_each: int) -> float:
    """Fraction of reserved slots left empty when every request reserves
    ``reserved_each`` contiguous slots up front (youngju.dev, waste example)."""
    reserved = reserved_each * len(used)
    return (reserved - sum(used)) / reserved


def paged_waste(used: Sequence[int], block_size: int = 16) -> float:
    """Fraction of allocated slots left empty when each request holds
    ceil(len / block_size) blocks: only the last block's tail can be empty
    (ta-paperlens, "fragmentation and PagedAttention")."""
    held = sum(-(-u // block_size) * block_size for u in used)
    return (held - sum(used)) / held if held else 0.0
