"""Pins for the oracle's block allocator and pool model (CPU only).

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/*.json, each with its citation), invariants the pages
state, or a brute-force replay of token histories.
"""
import json
import os
import random

import numpy as np
import pytest

from oracle import (BlockPoolModel, OutOfBlocks, PoolModel, contiguous_waste,
                    kv_bytes_per_token, kv_cache_size_gib, paged_waste)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_kv_bytes_per_token_printed_value():
    g = golden("kv_bytes_per_token.json")
    b = kv_bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["dtype_bytes"])
    assert b == g["bytes_per_token"] == 131072
    assert b == g["page_prints_kib"] * 1024
    # the page's rounded follow-on figures, within their rounding
    one = kv_cache_size_gib(g["layers"], g["kv_heads"], g["head_dim"], 2000, 1) * 1024
    assert abs(one - 256) / 256 < 0.03            # "256 MiB" for 2,000 tokens
    hundred = kv_cache_size_gib(g["layers"], g["kv_heads"], g["head_dim"], 2000, 100)
    assert abs(hundred - 25) / 25 < 0.03          # "25 GiB" for 100 requests
    assert b * 2000 == g["exact_bytes_2000_tokens"]
    assert b * 2048 == g["exact_bytes_2048_tokens"] == 256 * 2**20


def test_kv_size_function_example_is_a_documented_discrepancy():
    g = golden("kv_size_function_example.json")
    a = g["example_args"]
    gib = kv_cache_size_gib(a["layers"], a["heads"], a["head_dim"], a["seq_len"], a["batch"],
                            a["dtype_bytes"])
    assert gib == pytest.approx(10.0)
    gib8 = kv_cache_size_gib(a["layers"], 8, a["head_dim"], a["seq_len"], a["batch"],
                             a["dtype_bytes"])
    assert gib8 == pytest.approx(1.25)
    # the printed "about 5.2 GB" matches neither reading
    assert abs(gib - 5.2) > 1 and abs(gib8 - 5.2) > 1


def test_contiguous_waste_printed_example():
    g = golden("contiguous_waste_example.json")
    assert g["reserved_each"] * len(g["used"]) == g["total_reserved"]
    assert sum(g["used"]) == g["total_used"]
    assert contiguous_waste(g["used"], g["reserved_each"]) == pytest.approx(g["waste_fraction"])
    # paging: only the last block's tail can be empty; these lengths are
    # multiples of 16 so nothing is wasted
    assert paged_waste(g["used"]) == 0.0
    # and in general the waste is below one block per request
    rng = np.random.default_rng(0)
    used = rng.integers(1, 5000, size=50).tolist()
    held = sum(-(-u // 16) * 16 for u in used)
    assert held - sum(used) < 16 * len(used)
    assert paged_waste(used) == pytest.approx((held - sum(used)) / held)


def test_block_table_diagram():
    """Request R1 appends 4 blocks' worth of tokens, then R2 3 blocks'; a free
    list ordered so that pops come out 0, 3, 1, 4, 2, 5, 6 reproduces the
    diagram's placement, with physical block 7 still free."""
    g = golden("block_table_diagram.json")
    pool = BlockPoolModel(g["num_blocks"], 16, free_order=[7, 6, 5, 2, 4, 1, 3, 0])
    pool.add(1)
    pool.add(2)
    slots1, _ = pool.append([1], [64])
    slots2, _ = pool.append([2], [48])
    assert pool.table(1) == g["r1_table"]
    assert sorted(pool.table(2)) == g["r2_physical_positions"]
    assert pool.free == g["free_positions"]
    # logical token p of R1 sits in physical block table[p // 16] at offset p % 16
    for p, s in enumerate(slots1):
        assert s == g["r1_table"][p // 16] * 16 + p % 16
    pool.check()


def test_lifo_pop_from_end_and_push_to_end():
    pool = BlockPoolModel(4, 16)           # free list [0, 1, 2, 3]
    pool.add(0)
    pool.append([0], [1])
    assert pool.table(0) == [3]            # pop takes the last entry
    pool.add(1)
    pool.append([1], [17])
    assert pool.table(1) == [2, 1]
    pool.free_seq(1)                       # returned in logical order to the end
    assert pool.free == [0, 2, 1]
    pool.add(2)
    pool.append([2], [1])
    assert pool.table(2) == [1]


def test_out_of_blocks_is_an_error_and_changes_nothing():
    pool = BlockPoolModel(3, 16)
    pool.add(0)
    pool.add(1)
    pool.append([0], [32])
    before = (list(pool.free), list(pool.ref), {k: list(v) for k, v in pool.tables.items()},
              dict(pool.lens))
    with pytest.raises(OutOfBlocks):
        pool.append([1, 0], [16, 1])       # needs 2 blocks, 1 free
    after = (list(pool.free), list(pool.ref), {k: list(v) for k, v in pool.tables.items()},
             dict(pool.lens))
    assert before == after
    # preemption frees the newest request; the retry then fits
    pool.free_seq(0)
    pool.append([1], [16])
    pool.check()


def test_first_token_allocates_and_block_count_is_ceil():
    rng = random.Random(3)
    pool = BlockPoolModel(400, 16, free_order=np.random.default_rng(3).permutation(400))
    lens = {}
    for s in range(10):
        pool.add(s)
        lens[s] = 0
    for _ in range(60):
        s = rng.randrange(10)
        n = rng.randrange(0, 40)
        before_blocks = len(pool.table(s))
        slots, copies = pool.append([s], [n])
        lens[s] += n
        assert copies == []
        assert len(pool.table(s)) == -(-lens[s] // 16)
        new_blocks = len(pool.table(s)) - before_blocks
        assert new_blocks == sum(1 for x in slots if x % 16 == 0)
    pool.check()


def test_shared_prefix_example_ref_counts():
    g = golden("shared_prefix_example.json")
    pool = BlockPoolModel(16, 16)
    pool.add(0)
    pool.append([0], [16 * g["shared_blocks"]])
    for c in range(1, g["requests"]):
        pool.fork(0, c)
    shared = pool.table(0)
    for c in range(g["requests"]):
        pool.append([c], [5])
    for b in shared:
        assert pool.ref[b] == g["shared_ref_count"]
    privates = [pool.table(c)[g["shared_blocks"]] for c in range(g["requests"])]
    assert len(set(privates)) == g["requests"]
    assert all(pool.ref[b] == 1 for b in privates)
    assert all(pool.table(c)[:g["shared_blocks"]] == shared for c in range(g["requests"]))
    pool.check()


def test_copy_on_write_last_sharer_writes_in_place():
    pool = BlockPoolModel(8, 16)
    pool.add(0)
    pool.append([0], [20])                 # block 1 holds 4 tokens
    pool.fork(0, 1)
    pool.fork(0, 2)
    partial = pool.table(0)[1]
    assert pool.ref[partial] == 3
    assert pool.blocks_needed([0, 1, 2], [1, 1, 1]) == 2
    slots, copies = pool.append([0, 1, 2], [1, 1, 1])
    assert [c[0] for c in copies] == [partial, partial]
    assert [c[2] for c in copies] == [4, 4]
    assert pool.table(2)[1] == partial     # last sharer keeps the original
    assert pool.ref[partial] == 1
    assert slots[2] == partial * 16 + 4
    pool.check()


def _replay_random_program(seed, num_blocks=12, steps=80):
    """Random add/append/fork/free program; every append stores distinct
    random rows; returns (pool, model, histories).  The pages' promise: each
    request always sees exactly its own token history, however blocks are
    placed, shared or copied."""
    rng = np.random.default_rng(seed)
    pool = BlockPoolModel(num_blocks, 16, free_order=rng.permutation(num_blocks))
    mem = PoolModel(num_blocks, 2, 8)
    hist = {}
    next_id = 0
    for _ in range(steps):
        op = rng.integers(0, 6)
        live = sorted(hist)
        if op == 0 or not live:
            pool.add(next_id)
            hist[next_id] = (np.zeros((0, 2, 8), np.float16), np.zeros((0, 2, 8), np.float16))
            next_id += 1
        elif op == 1 and live:
            p = int(rng.choice(live))
            pool.fork(p, next_id)
            hist[next_id] = (hist[p][0].copy(), hist[p][1].copy())
            next_id += 1
        elif op == 2 and len(live) > 1:
            s = int(rng.choice(live))
            pool.free_seq(s)
            del hist[s]
        else:
            k = int(rng.integers(1, min(4, len(live)) + 1))
            ids = [int(x) for x in rng.choice(live, size=k, replace=False)]
            n = [int(x) for x in rng.integers(0, 20, size=k)]
            need = pool.blocks_needed(ids, n)
            free_before = pool.num_free()
            try:
                slots, copies = pool.append(ids, n)
            except OutOfBlocks:
                assert need > free_before
                continue
            assert free_before - pool.num_free() == need
            t = sum(n)
            kr = rng.standard_normal((t, 2, 8)).astype(np.float16)
            vr = rng.standard_normal((t, 2, 8)).astype(np.float16)
            mem.copy(copies)
            mem.write(kr, vr, slots)
            c = 0
            for s, m in zip(ids, n):
                hist[s] = (np.concatenate([hist[s][0], kr[c:c + m]]),
                           np.concatenate([hist[s][1], vr[c:c + m]]))
                c += m
        pool.check()
    return pool, mem, hist


@pytest.mark.parametrize("seed", range(12))
def test_every_request_sees_its_own_history(seed):
    pool, mem, hist = _replay_random_program(seed)
    for s, (k, v) in hist.items():
        gk, gv = mem.gather(pool.tables[s], pool.lens[s])
        assert np.array_equal(gk.view(np.uint16), k.view(np.uint16))
        assert np.array_equal(gv.view(np.uint16), v.view(np.uint16))


def test_live_slots_are_distinct_unless_shared():
    pool, _, hist = _replay_random_program(99, num_blocks=20, steps=120)
    owners = {}
    for s in hist:
        for p in range(pool.lens[s]):
            slot = pool.tables[s][p // 16] * 16 + p % 16
            owners.setdefault(slot, set()).add(s)
    for slot, who in owners.items():
        if len(who) > 1:
            assert pool.ref[slot // 16] >= len(who)
