"""Oracle model of the physical K/V pool bytes.  TEST INFRASTRUCTURE ONLY.

The pool is preallocated once as fp16 arrays (youngju.dev blog, the
PagedAttentionManager listing, which allocates K and V pools of the same shape
up front).  This model keeps both in plain logical order,

    K pool, V pool: [num_blocks][n_kv][16][d]   (one token row of d values per slot)

The device orders the values inside each (block, kv head) tile for its matrix
cores; the tests map device pools back to this order (by the layout rule the
C ABI header states) before comparing them bit for bit.

Writing a token (the listing's ``append_token`` store into
``cache[block, slot]``) and a copy-on-write copy (media.tcdigital.jp, memory
sharing section) are plain element copies, done here with explicit loops over
tokens and blocks.
"""
from __future__ import annotations

from typing import Iterable, Tuple

import numpy as np

from . import fp8


class PoolModel:
    def __init__(self, num_blocks: int, n_kv: int, d: int, block_size: int = 16):
        self.num_blocks, self.n_kv, self.d, self.bs = num_blocks, n_kv, d, block_size
        self.k = np.zeros((num_blocks, n_kv, block_size, d), dtype=np.float16)
        self.v = np.zeros((num_blocks, n_kv, block_size, d), dtype=np.float16)

    def write(self, k_rows: np.ndarray, v_rows: np.ndarray, slots: Iterable[int]) -> None:
        """Token t goes to slot ``slots[t]`` = block * 16 + offset; a negative
        slot means the token is not stored."""
        for t, s in enumerate(slots):
            s = int(s)
            if s < 0:
                continue
            blk, off = divmod(s, self.bs)
            self.k[blk, :, off, :] = k_rows[t]
            self.v[blk, :, off, :] = v_rows[t]

    def write_bulk(self, k_rows: np.ndarray, v_rows: np.ndarray, slots) -> None:
        """Same stores as ``write`` with numpy fancy indexing (large setups)."""
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        slots = slots[keep]
        blk, off = slots // self.bs, slots % self.bs
        self.k[blk, :, off, :] = k_rows[keep]
        self.v[blk, :, off, :] = v_rows[keep]

    def copy(self, copies: Iterable[Tuple[int, int, int]]) -> None:
        """Copy the first ``n`` slots of every KV head from ``src`` to ``dst``."""
        for src, dst, n in copies:
            self.k[dst, :, :n, :] = self.k[src, :, :n, :]
            self.v[dst, :, :n, :] = self.v[src, :, :n, :]

    def gather(self, table, length: int):
        """Logical K and V of one request, [length][n_kv][d] each, following
        its block table (logical block i lives in physical block table[i])."""
        k = np.empty((length, self.n_kv, self.d), dtype=np.float16)
        v = np.empty((length, self.n_kv, self.d), dtype=np.float16)
        for pos in range(0, length, self.bs):
            blk = table[pos // self.bs]
            n = min(self.bs, length - pos)
            k[pos:pos + n] = self.k[blk, :, :n, :].transpose(1, 0, 2)
            v[pos:pos + n] = self.v[blk, :, :n, :].transpose(1, 0, 2)
        return k, v

    def gather_values(self, table, length: int):
        """The logical K and V as fp64 values."""
        k, v = self.gather(table, length)
        return k.astype(np.float64), v.astype(np.float64)


class Fp8PoolModel(PoolModel):
    """The same pool holding one E4M3 code per value (the FP8 KV-cache
    variant): a stored row is ``fp8.quantize(row, scale)`` with one scale for
    the K pool and one for the V pool; copies and gathers move codes."""

    def __init__(self, num_blocks: int, n_kv: int, d: int, k_scale: float, v_scale: float,
                 block_size: int = 16):
        super().__init__(num_blocks, n_kv, d, block_size)
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.k = np.zeros((num_blocks, n_kv, block_size, d), dtype=np.uint8)
        self.v = np.zeros((num_blocks, n_kv, block_size, d), dtype=np.uint8)

    def write(self, k_rows, v_rows, slots) -> None:
        super().write(fp8.quantize(k_rows, self.k_scale), fp8.quantize(v_rows, self.v_scale),
                      slots)

    def write_bulk(self, k_rows, v_rows, slots) -> None:
        super().write_bulk(fp8.quantize(k_rows, self.k_scale), fp8.quantize(v_rows, self.v_scale),
                           slots)

    def gather(self, table, length: int):
        """Codes of one request's logical K and V, [length][n_kv][d] uint8."""
        k = np.empty((length, self.n_kv, self.d), dtype=np.uint8)
        v = np.empty((length, self.n_kv, self.d), dtype=np.uint8)
        for pos in range(0, length, self.bs):
            blk = table[pos // self.bs]
            n = min(self.bs, length - pos)
            k[pos:pos + n] = self.k[blk, :, :n, :].transpose(1, 0, 2)
            v[pos:pos + n] = self.v[blk, :, :n, :].transpose(1, 0, 2)
        return k, v

    def gather_values(self, table, length: int):
        """The fp64 values the codes stand for (code value times scale)."""
        k, v = self.gather(table, length)
        return fp8.dequantize(k, self.k_scale), fp8.dequantize(v, self.v_scale)
