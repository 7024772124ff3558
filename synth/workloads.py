"""Seeded synthetic workloads for paged decode attention and a chunked-prefill tile.

Every array here is drawn from ``numpy.random.default_rng(seed)`` and cast to
IEEE fp16 (round to nearest even).  Those fp16 arrays are the ground truth that
both the fp64 oracle and the HIP path consume; nothing in this module computes
attention or makes an allocation decision.  A workload is a small *program*
for the block manager (add / append / fork), the K/V rows that program appends,
and the inputs of one step (each decode sequence appends one token; in the
mixed configuration a prefill sequence appends a 512-token chunk).

Draw order, fixed so that every consumer sees the same bytes:
    lengths -> free-list permutation -> decode queries -> setup K -> setup V
    -> step K -> step V -> prefill-chunk queries.

Workload shapes follow the decode scenarios the pages use to motivate paging:
16-token blocks (ngrok summary, "PagedAttention" section; youngju.dev blog,
"PagedAttention" section), GQA with 8 KV heads and head_dim 128 (paperlens
explainer, KV-size example), a shared system-prompt prefix (youngju.dev blog,
copy-on-write section) and a 50,000-token prompt split into chunks (ngrok
summary, scheduler section).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK_SIZE = 16

CONFIG_NAMES = {
    "1": "tiny",
    "2": "llama3-8b-decode",
    "3": "llama3-70b-decode",
    "4": "prefix-sharing",
    "4b": "prefix-sharing-cow",
    "5": "long-context-mixed",
}

# A setup op is one of
#   ("add", seq_id)
#   ("append", [seq_ids], [n_new])        tokens taken in order from setup_k/v
#   ("fork", parent_id, child_id)
Op = Tuple


@dataclass
class PrefillChunk:
    seq_id: int
    q_start: int          # absolute position of the chunk's first query row
    chunk_len: int
    q: np.ndarray         # [chunk_len][n_q][d] fp16


@dataclass
class Workload:
    name: str
    n_q: int
    n_kv: int
    d: int
    scale: float
    num_blocks: int
    free_order: np.ndarray            # int32 [num_blocks]; free stack bottom -> top
    setup: List[Op]
    setup_k: np.ndarray               # [T_setup][n_kv][d] fp16, in append order
    setup_v: np.ndarray
    step_ids: np.ndarray              # int64, sequences appended to in the step
    step_n_new: np.ndarray            # int32, tokens each of them appends
    step_k: np.ndarray                # [T_step][n_kv][d] fp16
    step_v: np.ndarray
    decode_ids: np.ndarray            # int64 [B], sequences attended by decode
    q: np.ndarray                     # [B][n_q][d] fp16
    prefill: Optional[PrefillChunk] = None
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.decode_ids))

    @property
    def group(self) -> int:
        return self.n_q // self.n_kv


def _fp16(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a.astype(np.float16))


def _draw(rng: np.random.Generator, shape, dist: str) -> np.ndarray:
    """fp16 samples: 'uniform' is U[-1, 1] drawn in fp64; 'normal' is N(0, 1)
    drawn in fp32 (numpy's ziggurat) in slices to bound host memory."""
    if dist == "uniform":
        return _fp16(rng.uniform(-1.0, 1.0, size=shape))
    if dist != "normal":
        raise ValueError(dist)
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.float16)
    if len(shape) == 0 or shape[0] == 0:
        return out
    rows = shape[0]
    per_row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    step = max(1, (1 << 25) // max(per_row, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = rng.standard_normal((r1 - r0,) + shape[1:], dtype=np.float32)
    return out


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def _pool_size(blocks_needed: int, headroom: float = 0.10, extra: int = 0) -> int:
    return int(math.ceil(blocks_needed * (1.0 + headroom))) + extra


def _decode_only(name, seed, rng, lengths, n_q, n_kv, d, dist, num_blocks,
                 scale=None) -> Workload:
    """Each sequence i holds lengths[i]-1 cached tokens and appends one; the
    attended length is lengths[i] (the new token attends to itself).  ``rng``
    has already produced the lengths (or they are fixed)."""
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.min() >= 1
    B = len(lengths)
    free_order = rng.permutation(num_blocks).astype(np.int32)
    q = _draw(rng, (B, n_q, d), dist)
    cached = lengths - 1
    t_setup = int(cached.sum())
    setup_k = _draw(rng, (t_setup, n_kv, d), dist)
    setup_v = _draw(rng, (t_setup, n_kv, d), dist)
    step_k = _draw(rng, (B, n_kv, d), dist)
    step_v = _draw(rng, (B, n_kv, d), dist)
    ids = np.arange(B, dtype=np.int64)
    setup: List[Op] = [("add", int(i)) for i in ids]
    setup.append(("append", ids.tolist(), cached.astype(np.int32).tolist()))
    return Workload(
        name=name, n_q=n_q, n_kv=n_kv, d=d,
        scale=(1.0 / math.sqrt(d)) if scale is None else scale,
        num_blocks=num_blocks, free_order=free_order, setup=setup,
        setup_k=setup_k, setup_v=setup_v,
        step_ids=ids.copy(), step_n_new=np.ones(B, dtype=np.int32),
        step_k=step_k, step_v=step_v, decode_ids=ids.copy(), q=q, seed=seed,
        notes={"lengths": lengths.tolist()},
    )


def make_tiny_workload(lengths: Sequence[int], n_q: int = 4, n_kv: int = 2, d: int = 64,
                       num_blocks: Optional[int] = None, seed: int = 7,
                       dist: str = "uniform", scale: Optional[float] = None,
                       name: str = "custom") -> Workload:
    """A decode-only workload with caller-chosen attended lengths (tests)."""
    lengths = [int(x) for x in lengths]
    if num_blocks is None:
        num_blocks = _pool_size(sum(_ceil_div(x, BLOCK_SIZE) for x in lengths), extra=2)
    return _decode_only(name, seed, np.random.default_rng(seed), lengths, n_q, n_kv, d,
                        dist, num_blocks, scale)


def _cfg1() -> Workload:
    # 4 sequences, attended lengths {5, 16, 17, 33}; GQA 4/2; d 64; U[-1,1];
    # a 16-block pool whose free list is a seeded permutation.
    return _decode_only(CONFIG_NAMES["1"], 1001, np.random.default_rng(1001),
                        [5, 16, 17, 33], 4, 2, 64, "uniform", 16, scale=1.0 / 8.0)


def _cfg2() -> Workload:
    seed = 1002
    rng = np.random.default_rng(seed)
    lengths = rng.integers(128, 2048, size=64, endpoint=True)
    nb = _pool_size(int(sum(_ceil_div(int(x), BLOCK_SIZE) for x in lengths)))
    return _decode_only(CONFIG_NAMES["2"], seed, rng, lengths, 32, 8, 128, "normal", nb)


def _cfg3() -> Workload:
    seed = 1003
    rng = np.random.default_rng(seed)
    lengths = np.clip(np.rint(rng.lognormal(math.log(1000.0), 1.0, size=256)), 16, 4096)
    lengths = lengths.astype(np.int64)
    nb = _pool_size(int(sum(_ceil_div(int(x), BLOCK_SIZE) for x in lengths)))
    return _decode_only(CONFIG_NAMES["3"], seed, rng, lengths, 64, 8, 128, "normal", nb)


def _cfg4(cow_variant: bool) -> Workload:
    """128 requests share a prefix held by request 0 and forked to the rest.

    Plain variant: 1,024-token prefix (64 full blocks), then every request
    appends a private suffix of U{16..512} tokens, then the step appends one
    token each.  CoW variant: a 1,032-token prefix (block 64 half full and
    shared by all 128), no suffix, and the step's appends hit that block."""
    seed = 1004 if not cow_variant else 1014
    rng = np.random.default_rng(seed)
    B, n_q, n_kv, d = 128, 32, 8, 128
    prefix = 1032 if cow_variant else 1024
    if cow_variant:
        suffix = np.zeros(B, dtype=np.int64)
    else:
        suffix = rng.integers(16, 512, size=B, endpoint=True).astype(np.int64)
    lengths = prefix + suffix + 1
    full_shared = prefix // BLOCK_SIZE
    unique_blocks = full_shared + int(
        sum(_ceil_div(int(x), BLOCK_SIZE) - full_shared for x in lengths))
    nb = _pool_size(unique_blocks, extra=B if cow_variant else 0)
    free_order = rng.permutation(nb).astype(np.int32)
    q = _draw(rng, (B, n_q, d), "normal")
    t_setup = prefix + int(suffix.sum())
    setup_k = _draw(rng, (t_setup, n_kv, d), "normal")
    setup_v = _draw(rng, (t_setup, n_kv, d), "normal")
    step_k = _draw(rng, (B, n_kv, d), "normal")
    step_v = _draw(rng, (B, n_kv, d), "normal")
    ids = np.arange(B, dtype=np.int64)
    setup: List[Op] = [("add", 0), ("append", [0], [prefix])]
    for c in range(1, B):
        setup.append(("fork", 0, c))
    if suffix.sum() > 0:
        setup.append(("append", ids.tolist(), suffix.astype(np.int32).tolist()))
    return Workload(
        name=CONFIG_NAMES["4b" if cow_variant else "4"], n_q=n_q, n_kv=n_kv, d=d,
        scale=1.0 / math.sqrt(d), num_blocks=nb, free_order=free_order, setup=setup,
        setup_k=setup_k, setup_v=setup_v, step_ids=ids.copy(),
        step_n_new=np.ones(B, dtype=np.int32), step_k=step_k, step_v=step_v,
        decode_ids=ids.copy(), q=q, seed=seed,
        notes={"lengths": lengths.tolist(), "prefix": prefix,
               "unique_blocks_after_step": unique_blocks},
    )


def _cfg5() -> Workload:
    """8 decode sequences at attended length 32,768 plus one prompt of 50,000
    tokens whose last 512-token chunk (positions 49,488..49,999) is prefilled
    in the same step over the same pool."""
    seed = 1005
    rng = np.random.default_rng(seed)
    B, n_q, n_kv, d = 8, 32, 8, 128
    L, prompt, C = 32768, 50000, 512
    P0 = prompt - C
    blocks = B * _ceil_div(L, BLOCK_SIZE) + _ceil_div(prompt, BLOCK_SIZE)
    nb = _pool_size(blocks)
    free_order = rng.permutation(nb).astype(np.int32)
    q = _draw(rng, (B, n_q, d), "normal")
    t_setup = B * (L - 1) + P0
    setup_k = _draw(rng, (t_setup, n_kv, d), "normal")
    setup_v = _draw(rng, (t_setup, n_kv, d), "normal")
    step_k = _draw(rng, (B + C, n_kv, d), "normal")
    step_v = _draw(rng, (B + C, n_kv, d), "normal")
    q_chunk = _draw(rng, (C, n_q, d), "normal")
    dec = np.arange(B, dtype=np.int64)
    pid = B
    setup: List[Op] = [("add", int(i)) for i in range(B + 1)]
    setup.append(("append", dec.tolist() + [pid], [L - 1] * B + [P0]))
    return Workload(
        name=CONFIG_NAMES["5"], n_q=n_q, n_kv=n_kv, d=d, scale=1.0 / math.sqrt(d),
        num_blocks=nb, free_order=free_order, setup=setup,
        setup_k=setup_k, setup_v=setup_v,
        step_ids=np.concatenate([dec, [pid]]).astype(np.int64),
        step_n_new=np.array([1] * B + [C], dtype=np.int32),
        step_k=step_k, step_v=step_v, decode_ids=dec, q=q,
        prefill=PrefillChunk(seq_id=pid, q_start=P0, chunk_len=C, q=q_chunk),
        seed=seed,
        notes={"lengths": [L] * B, "prompt": prompt},
    )


def make_workload(cfg) -> Workload:
    """Build configuration ``cfg`` in {1, 2, 3, 4, '4b', 5}."""
    key = str(cfg)
    if key == "1":
        return _cfg1()
    if key == "2":
        return _cfg2()
    if key == "3":
        return _cfg3()
    if key == "4":
        return _cfg4(False)
    if key == "4b":
        return _cfg4(True)
    if key == "5":
        return _cfg5()
    raise KeyError(cfg)


def make_mixed_workload(decode_lengths: Sequence[int], q_start: int, chunk_len: int,
                        n_q: int = 32, n_kv: int = 8, d: int = 128, seed: int = 11,
                        dist: str = "normal", num_blocks: Optional[int] = None,
                        name: str = "mixed") -> Workload:
    """Decode requests of the given attended lengths plus one prompt whose
    chunk [q_start, q_start + chunk_len) is prefilled in the same step (the
    shape of configuration 5 at any size; tests)."""
    rng = np.random.default_rng(seed)
    lengths = np.asarray(list(decode_lengths), dtype=np.int64)
    B = len(lengths)
    blocks = int(sum(_ceil_div(int(x), BLOCK_SIZE) for x in lengths)) + \
        _ceil_div(q_start + chunk_len, BLOCK_SIZE)
    nb = _pool_size(blocks, extra=2) if num_blocks is None else num_blocks
    free_order = rng.permutation(nb).astype(np.int32)
    q = _draw(rng, (B, n_q, d), dist)
    t_setup = int((lengths - 1).sum()) + q_start
    setup_k = _draw(rng, (t_setup, n_kv, d), dist)
    setup_v = _draw(rng, (t_setup, n_kv, d), dist)
    step_k = _draw(rng, (B + chunk_len, n_kv, d), dist)
    step_v = _draw(rng, (B + chunk_len, n_kv, d), dist)
    q_chunk = _draw(rng, (chunk_len, n_q, d), dist)
    dec = np.arange(B, dtype=np.int64)
    pid = B
    setup: List[Op] = [("add", int(i)) for i in range(B + 1)]
    setup.append(("append", dec.tolist() + [pid], (lengths - 1).astype(int).tolist() + [q_start]))
    return Workload(
        name=name, n_q=n_q, n_kv=n_kv, d=d, scale=1.0 / math.sqrt(d), num_blocks=nb,
        free_order=free_order, setup=setup, setup_k=setup_k, setup_v=setup_v,
        step_ids=np.concatenate([dec, [pid]]).astype(np.int64),
        step_n_new=np.array([1] * B + [chunk_len], dtype=np.int32),
        step_k=step_k, step_v=step_v, decode_ids=dec, q=q,
        prefill=PrefillChunk(seq_id=pid, q_start=q_start, chunk_len=chunk_len, q=q_chunk),
        seed=seed, notes={"lengths": lengths.tolist(), "prompt": q_start + chunk_len},
    )
