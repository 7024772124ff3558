"""Oracle model of prefix caching on top of the block pool model.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What it follows:
  * ngrok summary, "prefix caching" section: requests that start with the
    same tokens share the KV data of that common part instead of computing
    it again; the condition is the same token sequence at the same
    positions, so one differing token ends the sharing for everything after
    it; sharing is decided block by block, each block being identified by
    its own tokens together with (the hash of) everything before it.
  * youngju.dev blog, "copy-on-write prefix sharing" listing: the blocks of
    a shared system prompt carry a reference count equal to the number of
    requests using them, each request's own tokens live in private blocks.
  * ta-paperlens, "fragmentation and PagedAttention": physical blocks can be
    shared; writes into a shared block copy it first.

Readings (the pages leave these open):
  * Only full blocks (16 tokens) are cached; the identity of block i of a
    prompt is the whole token prefix 0 .. 16(i+1)-1.  The model keys blocks
    by that exact tuple (the library keys them by a hash chain and checks
    the parent hash and the block's tokens on a hit).
  * A block enters the cache when the caller registers the tokens of a
    sequence (``register``): its full blocks get their prefix keys, in
    order.  A key already held by another block stays with that block.
  * ``add_cached`` starts a new sequence from the longest run of cached
    blocks matching the prompt from its first token; a hit takes one more
    reference (the same sharing as ``fork``).  The new sequence's length is
    16 * hits; the caller appends the remaining tokens as usual.
  * A block whose last reference goes away keeps its key and becomes
    evictable instead of free.  Allocation takes never-cached free blocks
    first (the pool's LIFO stack); only when none is left does it evict the
    evictable block that became evictable longest ago, dropping its key.
    A hit on an evictable block revives it.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

from .allocator import BlockPoolModel, OutOfBlocks


class PrefixCachingPoolModel(BlockPoolModel):
    def __init__(self, num_blocks: int, block_size: int = 16, free_order=None):
        super().__init__(num_blocks, block_size, free_order)
        self.cache: Dict[Tuple[int, ...], int] = {}   # prefix tokens -> block
        self.key_of: Dict[int, Tuple[int, ...]] = {}  # block -> its prefix key
        self.evictable: List[int] = []                # oldest first

    # -- allocation ----------------------------------------------------------
    def _available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            b = self.free.pop()
        else:
            b = self.evictable.pop(0)
            del self.cache[self.key_of.pop(b)]
        self.ref[b] = 1
        return b

    def append(self, ids: Sequence[int], n_new: Sequence[int]):
        """As ``BlockPoolModel.append``, with eviction when the free list is
        empty (new blocks and copy-on-write targets come from ``_take``)."""
        need = self._plan(ids, n_new)
        if need > self._available():
            raise OutOfBlocks(f"need {need} blocks, {self._available()} available")
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
                    blk = self._take()
                    table.append(blk)
                else:
                    blk = table[logical]
                    if self.ref[blk] > 1:
                        new = self._take()
                        self.ref[blk] -= 1
                        copies.append((blk, new, off))
                        table[logical] = new
                        blk = new
                slots.append(blk * self.block_size + off)
                self.lens[seq] = pos + 1
        return slots, copies

    def num_free(self) -> int:
        return self._available()

    # -- release -------------------------------------------------------------
    def free_seq(self, seq: int) -> None:
        table = self.tables.pop(seq)
        del self.lens[seq]
        for b in table:
            self.ref[b] -= 1
            if self.ref[b] == 0:
                if b in self.key_of:
                    self.evictable.append(b)
                else:
                    self.free.append(b)

    # -- the cache -----------------------------------------------------------
    def register(self, seq: int, tokens: Sequence[int]) -> int:
        """Give the full blocks of ``seq`` covered by ``tokens`` (its first
        len(tokens) token ids) their prefix keys.  Returns how many blocks
        were newly registered."""
        tokens = [int(t) for t in tokens]
        if len(tokens) > self.lens[seq]:
            raise ValueError("more tokens than the sequence holds")
        bs = self.block_size
        added = 0
        for i in range(len(tokens) // bs):
            blk = self.tables[seq][i]
            key = tuple(tokens[:bs * (i + 1)])
            if blk in self.key_of or key in self.cache:
                continue
            self.cache[key] = blk
            self.key_of[blk] = key
            added += 1
        return added

    def add_cached(self, seq: int, tokens: Sequence[int]) -> int:
        """New sequence whose table starts with the cached blocks matching
        ``tokens`` from the first token on.  Returns the cached token count."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        table: List[int] = []
        for i in range(len(tokens) // bs):
            blk = self.cache.get(tuple(tokens[:bs * (i + 1)]))
            if blk is None:
                break
            if self.ref[blk] == 0:
                self.evictable.remove(blk)
            self.ref[blk] += 1
            table.append(blk)
        self.tables[seq] = table
        self.lens[seq] = bs * len(table)
        return bs * len(table)

    # -- invariants ------------------------------------------------------------
    def check(self) -> None:
        held = [0] * self.num_blocks
        for seq, t in self.tables.items():
            assert len(t) == -(-self.lens[seq] // self.block_size), seq
            for b in t:
                held[b] += 1
        assert held == self.ref
        free, ev = set(self.free), set(self.evictable)
        assert len(free) == len(self.free) and len(ev) == len(self.evictable)
        assert not (free & ev)
        for b in range(self.num_blocks):
            if self.ref[b] == 0:
                assert (b in free) != (b in ev), b
            else:
                assert b not in free and b not in ev, b
        for b in ev:
            assert b in self.key_of
        for b in free:
            assert b not in self.key_of
        assert len(self.cache) == len(self.key_of)
        for key, b in self.cache.items():
            assert self.key_of[b] == key and len(key) % self.block_size == 0
