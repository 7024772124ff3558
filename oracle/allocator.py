"""Oracle model of the physical KV block pool and per-request block tables.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What it follows:
  * youngju.dev blog, "PagedAttention" section (the PagedAttentionManager
    listing): the free list starts as every block id, allocation takes the
    last entry, an empty list is an error, a freed block goes back on the end,
    and a request gets a new block when its token count is a multiple of the
    block size.  Read here as a LIFO stack; the very first token of an empty
    request also allocates (the listing presumes a non-empty table).
  * ngrok summary, "PagedAttention" section: no up-front reservation; a new
    block only when the last one is full; blocks may live anywhere; a table
    maps each request's data to blocks.
  * media.tcdigital.jp, "memory sharing for parallel sampling": prompt blocks
    are shared by reference and a new block is allocated only when outputs
    diverge (copy-on-write).  Read here as: ``fork`` shares every block
    (reference count + 1); appending into a partially filled block whose
    reference count is above one first copies the filled slots into a fresh
    block; the last remaining sharer writes in place.
  * youngju.dev blog, copy-on-write section: shared blocks carry a
    reference count equal to the number of requests using them.

Sequences in one append call are processed in the order given; a sequence's
tokens are processed in position order.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional, Sequence, Tuple


class OutOfBlocks(Exception):
    """The free list cannot cover the request (state is left unchanged)."""


class BlockPoolModel:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Iterable[int]] = None):
        if block_size != 16:
            raise ValueError("block size is fixed at 16 tokens")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if free_order is None:
            self.free: List[int] = list(range(self.num_blocks))
        else:
            self.free = [int(x) for x in free_order]
            if sorted(self.free) != list(range(self.num_blocks)):
                raise ValueError("free_order must be a permutation of the block ids")
        self.ref: List[int] = [0] * self.num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- sequences -----------------------------------------------------------
    def add(self, seq: int) -> None:
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables:
            raise KeyError(f"unknown sequence {parent}")
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int) -> None:
        """Drop one reference to each block, in logical order; a block whose
        count reaches zero returns to the end of the free list."""
        table = self.tables.pop(seq)
        del self.lens[seq]
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- appending -----------------------------------------------------------
    def _plan(self, ids: Sequence[int], n_new: Sequence[int]) -> int:
        """Blocks the append would take off the free list (new blocks plus
        copy-on-write targets), simulated without touching the state."""
        if len(set(int(s) for s in ids)) != len(ids):
            raise ValueError("duplicate sequence id in one append")
        sim_ref: Dict[int, int] = {}
        need = 0
        for seq, n in zip(ids, n_new):
            seq, n = int(seq), int(n)
            if seq not in self.tables:
                raise KeyError(f"unknown sequence {seq}")
            if n < 0:
                raise ValueError("negative token count")
            if n == 0:
                continue
            length = self.lens[seq]
            off = length % self.block_size
            if off != 0:
                blk = self.tables[seq][length // self.block_size]
                r = sim_ref.get(blk, self.ref[blk])
                if r > 1:
                    need += 1
                    sim_ref[blk] = r - 1
            first_new = length if off == 0 else length + (self.block_size - off)
            end = length + n
            if end > first_new:
                need += -(-(end - first_new) // self.block_size)
        return need

    def blocks_needed(self, ids: Sequence[int], n_new: Sequence[int]) -> int:
        return self._plan(ids, n_new)

    def append(self, ids: Sequence[int], n_new: Sequence[int]
               ) -> Tuple[List[int], List[Tuple[int, int, int]]]:
        """Reserve slots for ``n_new[i]`` tokens of sequence ``ids[i]``.

        Returns (slot_mapping, copies): one slot per new token in (sequence,
        position) order, slot = physical_block * 16 + offset; and the
        copy-on-write list of (src_block, dst_block, filled_slots)."""
        need = self._plan(ids, n_new)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        slots: List[int] = []
        copies: List[Tuple[int, int, int]] = []
        for seq, n in zip(ids, n_new):
            seq, n = int(seq), int(n)
            table = self.tables[seq]
            for _ in range(n):
                pos = self.lens[seq]
                off = pos % self.block_size
                logical = pos // self.block_size
                if off == 0:
                    blk = self.free.pop()
                    self.ref[blk] = 1
                    table.append(blk)
                else:
                    blk = table[logical]
                    if self.ref[blk] > 1:
                        new = self.free.pop()
                        self.ref[new] = 1
                        self.ref[blk] -= 1
                        copies.append((blk, new, off))
                        table[logical] = new
                        blk = new
                slots.append(blk * self.block_size + off)
                self.lens[seq] = pos + 1
        return slots, copies

    # -- views ---------------------------------------------------------------
    def table(self, seq: int) -> List[int]:
        return list(self.tables[seq])

    def block_tables(self, ids: Sequence[int], max_blocks: int):
        rows, lens = [], []
        for s in ids:
            t = self.tables[int(s)]
            if len(t) > max_blocks:
                raise ValueError("table longer than max_blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lens[int(s)])
        return rows, lens

    def num_free(self) -> int:
        return len(self.free)

    def check(self) -> None:
        """free + referenced == N; each block's count equals the number of
        tables holding it; every table has ceil(len / 16) entries."""
        held = [0] * self.num_blocks
        for seq, t in self.tables.items():
            assert len(t) == -(-self.lens[seq] // self.block_size), seq
            for b in t:
                held[b] += 1
        assert held == self.ref
        assert len(set(self.free)) == len(self.free)
        for b in self.free:
            assert self.ref[b] == 0
        assert len(self.free) + sum(1 for r in self.ref if r > 0) == self.num_blocks
