"""Pins of the prefix-caching oracle (CPU only).

Each test checks the model against something fixed outside it: the worked
example the pages print, a closed form of the pages' sharing rule, or a
brute-force longest-common-prefix search over the registered prompts.
"""
import json
import os

import numpy as np
import pytest

from oracle.allocator import OutOfBlocks
from oracle.prefix_cache import PrefixCachingPoolModel

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def start(m, seq, tokens):
    """A request's prefill: take what the cache has, append and register the rest."""
    hit = m.add_cached(seq, tokens)
    m.append([seq], [len(tokens) - hit])
    m.register(seq, tokens)
    m.check()
    return hit


def test_system_prompt_blocks_shared_by_three_requests():
    # youngju.dev, copy-on-write prefix sharing: three requests with the same
    # system prompt share its blocks 0..2 (ref_count 3), each has one more
    # block of its own
    g = golden("shared_prefix_example.json")
    m = PrefixCachingPoolModel(32)
    rng = np.random.default_rng(0)
    system = [int(t) for t in rng.integers(0, 50000, size=16 * g["shared_blocks"])]
    hits = []
    for r in range(g["requests"]):
        suffix = [100000 + 10 * r + i for i in range(7)]
        hits.append(start(m, r, system + suffix))
    assert hits == [0] + [16 * g["shared_blocks"]] * (g["requests"] - 1)
    tables = [m.table(r) for r in range(g["requests"])]
    shared = tables[0][:g["shared_blocks"]]
    for t in tables:
        assert t[:g["shared_blocks"]] == shared
        assert len(t) - g["shared_blocks"] == g["private_blocks_each"]
    assert [m.ref[b] for b in shared] == [g["shared_ref_count"]] * g["shared_blocks"]
    private = [t[-1] for t in tables]
    assert len(set(private)) == g["requests"] and all(m.ref[b] == 1 for b in private)


def test_one_differing_token_ends_sharing_from_its_block():
    # ngrok summary, prefix caching: same tokens at the same positions; one
    # differing token and nothing after it is shared -> 16 * (p // 16)
    rng = np.random.default_rng(1)
    base = [int(t) for t in rng.integers(0, 1000, size=80)]
    for p in range(80):
        m = PrefixCachingPoolModel(16)
        start(m, 0, base)
        other = list(base)
        other[p] = 5000
        assert m.add_cached(1, other) == 16 * (p // 16), p
        m.check()


def test_same_tokens_at_another_position_are_not_shared():
    rng = np.random.default_rng(2)
    a = [int(t) for t in rng.integers(0, 1000, size=48)]
    m = PrefixCachingPoolModel(16)
    start(m, 0, a)
    assert m.add_cached(1, [7] * 16 + a[:32]) == 0          # a's block 0 moved to block 1
    assert m.add_cached(2, [7] + a[:47]) == 0               # shifted by one token
    assert m.add_cached(3, a[:40]) == 32                     # a prefix of a: its full blocks
    m.check()


def lcp(x, y):
    n = 0
    while n < min(len(x), len(y)) and x[n] == y[n]:
        n += 1
    return n


@pytest.mark.parametrize("seed", range(4))
def test_hits_equal_brute_force_longest_common_prefix(seed):
    rng = np.random.default_rng(10 + seed)
    m = PrefixCachingPoolModel(400)
    stems = [[int(t) for t in rng.integers(0, 2, size=48)] for _ in range(3)]
    registered = []
    for s in range(12):
        stem = stems[int(rng.integers(0, 3))]
        cut = int(rng.integers(0, 49))
        toks = stem[:cut] + [int(t) for t in rng.integers(0, 2, size=int(rng.integers(0, 40)))]
        start(m, s, toks)
        registered.append((s, toks))
    for q in range(40):
        stem = stems[int(rng.integers(0, 3))]
        cut = int(rng.integers(0, 49))
        prompt = stem[:cut] + [int(t) for t in rng.integers(0, 2, size=int(rng.integers(0, 40)))]
        # brute force: the longest run of whole blocks some registered prompt has in common
        best, owner = 0, None
        for s, toks in registered:
            k = min(lcp(prompt, toks), len(toks)) // 16
            if k > best:
                best, owner = k, s
        hit = m.add_cached(100 + q, prompt)
        assert hit == 16 * best
        if owner is not None:
            assert m.table(100 + q) == m.table(owner)[:best]
        m.free_seq(100 + q)
        m.check()


def test_eviction_takes_free_blocks_first_then_the_oldest_evictable():
    m = PrefixCachingPoolModel(8, free_order=list(range(8)))
    A, B, C = [1] * 32, [2] * 32, [3] * 32
    for s, t in ((0, A), (1, B), (2, C)):
        start(m, s, t)
    a, b, c = m.table(0), m.table(1), m.table(2)
    m.free_seq(0)
    m.free_seq(2)
    m.free_seq(1)                              # evictable, oldest first: a, c, b
    assert m.evictable == a + c + b and len(m.free) == 2
    m.add(3)
    m.append([3], [64])                        # 4 blocks: the 2 free ones, then a's
    assert set(a) <= set(m.table(3)) and not (set(m.table(3)) & set(b + c))
    assert m.add_cached(4, A) == 0             # evicted
    assert m.add_cached(5, C) == 32 and m.table(5) == c   # revived
    assert m.add_cached(6, B) == 32 and m.table(6) == b
    assert m.evictable == [] and m.num_free() == 0
    with pytest.raises(OutOfBlocks):
        m.append([4], [1])
    m.check()


def test_free_keeps_registered_blocks_and_hit_revives_them():
    m = PrefixCachingPoolModel(6)
    t = list(range(40))                        # 2 full blocks + 8 tokens
    start(m, 0, t)
    blocks = m.table(0)
    m.free_seq(0)
    assert m.evictable == blocks[:2] and blocks[2] in m.free   # the partial block was never cached
    assert m.num_free() == 6
    assert m.add_cached(1, t) == 32 and m.table(1) == blocks[:2]
    assert m.evictable == [] and [m.ref[b] for b in blocks[:2]] == [1, 1]
    m.check()
