"""Pins of the scheduler oracle (CPU only): the pages' rules written as
closed forms (decode first, chunked prefill of a 50,000-token prompt,
preempting the request added last) and invariants on random traces."""
import numpy as np
import pytest

from oracle.allocator import BlockPoolModel
from oracle.scheduler import SchedulerModel


def run_to_end(s, max_steps=100000):
    steps = []
    while s.waiting or s.running or s.swapped:
        steps.append(s.schedule())
        s.commit()
        assert len(steps) < max_steps
    return steps


def test_decode_first_within_the_budget():
    # ngrok, scheduler: running (decoding) requests first, prefill only with
    # budget left over
    s = SchedulerModel(BlockPoolModel(64), token_budget=3, max_running=8)
    for rid in range(3):
        s.add_request(rid, prompt=1, out=10)
    p = s.schedule(); s.commit()                 # three one-token prefills
    assert [i[:3] for i in p.items] == [(0, 0, 1), (1, 0, 1), (2, 0, 1)]
    s.add_request(9, prompt=5, out=1)
    p = s.schedule(); s.commit()
    assert [(i[0], i[2], i[3]) for i in p.items] == [(0, 1, 1), (1, 1, 1), (2, 1, 1)]
    assert p.admitted == [] and list(s.waiting) == [9]
    s2 = SchedulerModel(BlockPoolModel(64), token_budget=5, max_running=8)
    for rid in range(3):
        s2.add_request(rid, prompt=1, out=10)
    s2.schedule(); s2.commit()
    s2.add_request(9, prompt=5, out=1)
    p = s2.schedule()                            # 3 decodes, then 2 prefill tokens of 9
    assert [(i[0], i[1], i[2]) for i in p.items] == [(0, 1, 1), (1, 1, 1), (2, 1, 1), (9, 0, 2)]


def test_long_prompt_is_chunked_to_the_budget():
    # ngrok, scheduler: a 50,000-token prompt is split into budget-sized
    # chunks over several passes
    s = SchedulerModel(BlockPoolModel(4000), token_budget=2048, max_running=4)
    s.add_request(0, prompt=50000, out=3)
    steps = run_to_end(s)
    sizes = [p.items[0][2] for p in steps]
    assert sizes == [2048] * 24 + [50000 - 24 * 2048] + [1, 1]
    assert [p.items[0][1] for p in steps[:25]] == [2048 * k for k in range(25)]


def test_unconstrained_requests_finish_after_prefill_plus_outputs():
    # no memory or budget pressure: a request admitted at step a finishes at
    # step a + out - 1 (its prefill step yields the first token)
    s = SchedulerModel(BlockPoolModel(10000), token_budget=100000, max_running=100)
    rng = np.random.default_rng(0)
    arrive = {}
    finish = {}
    step = 0
    rid = 0
    while step < 60 or s.running or s.waiting:
        if step < 60:
            for _ in range(int(rng.integers(0, 3))):
                s.add_request(rid, prompt=int(rng.integers(1, 300)), out=int(rng.integers(1, 20)))
                arrive[rid] = step
                rid += 1
        s.schedule()
        for f in s.commit():
            finish[f] = step
        step += 1
    for r, a in arrive.items():
        assert finish[r] == a + s.reqs[r].out - 1, r


def test_preemption_takes_the_request_added_last_and_recomputes_it():
    # ngrok, scheduler: when blocks run out the most recently added request
    # is preempted, returns to the head of the waiting queue and is computed
    # again later; ta-paperlens skeleton: preempt(running[-1])
    pool = BlockPoolModel(5)
    s = SchedulerModel(pool, token_budget=64, max_running=8)
    s.add_request(0, prompt=32, out=40)          # 2 blocks, grows
    s.add_request(1, prompt=32, out=40)
    p = s.schedule(); s.commit()
    assert p.admitted == [0, 1] and pool.num_free() == 1
    preempted = []
    for _ in range(20):
        p = s.schedule()
        preempted += p.preempted
        s.commit()
        if preempted:
            break
    assert preempted == [1]
    assert s.reqs[1].computed == 0 and list(s.waiting)[0] == 1
    assert 1 not in s.running and 0 in s.running
    run_to_end(s)
    assert sorted(s.finished) == [0, 1] and pool.num_free() == 5
    assert s.reqs[1].preemptions >= 1 and s.reqs[0].preemptions == 0


@pytest.mark.parametrize("seed", range(5))
def test_random_traces_keep_the_invariants(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(20, 80))
    pool = BlockPoolModel(n, 16, rng.permutation(n))
    budget = int(rng.integers(8, 200))
    s = SchedulerModel(pool, token_budget=budget, max_running=int(rng.integers(1, 12)))
    rid = 0
    processed = {}
    for step in range(400):
        if step < 200:
            for _ in range(int(rng.integers(0, 3))):
                prompt = int(rng.integers(1, 16 * max(1, n // 4)))
                s.add_request(rid, prompt=prompt, out=int(rng.integers(1, 30)))
                rid += 1
        p = s.schedule()
        assert sum(i[2] for i in p.items) <= budget
        assert len(p.slots) == sum(i[2] for i in p.items)
        assert not (set(s.running) & set(s.waiting))
        for r_, start, k, _ in p.items:
            processed[r_] = processed.get(r_, 0) + k
        s.commit()
        pool.check()
        if not s.waiting and not s.running and step >= 200:
            break
    for p in run_to_end(s):
        for r_, start, k, _ in p.items:
            processed[r_] = processed.get(r_, 0) + k
    assert sorted(s.finished) == list(range(rid))
    assert pool.num_free() == n
    for r in s.reqs.values():                    # every input token computed at least once
        assert processed[r.rid] >= r.prompt + r.out - 1


def test_swap_preemption_keeps_the_victims_progress():
    # ta-paperlens skeleton: preempt(running[-1]), moved to CPU memory instead
    # of dropped; it resumes where it stopped, recomputing nothing
    pool = BlockPoolModel(5)
    s = SchedulerModel(pool, token_budget=64, max_running=8, swap=True)
    s.add_request(0, prompt=32, out=40)
    s.add_request(1, prompt=32, out=40)
    p = s.schedule(); s.commit()
    assert p.admitted == [0, 1] and pool.num_free() == 1
    for _ in range(20):
        table1, len1 = list(pool.tables[1]), s.reqs[1].computed
        p = s.schedule()
        if p.preempted:
            break
        s.commit()
    assert p.preempted == [1] and p.swap_out == [(1, table1, len1)]
    assert s.reqs[1].computed == len1 > 0 and list(s.swapped) == [1] and not s.waiting
    assert 1 not in s.running and 1 not in pool.tables
    s.commit()
    resumed = None
    while resumed is None:
        p = s.schedule()
        for rid, blocks, ln in p.swap_in:
            resumed = (rid, blocks, ln)
        s.commit()
    assert resumed[0] == 1 and resumed[2] == len1 and len(resumed[1]) == -(-len1 // 16)
    steps = run_to_end(s)
    assert sorted(s.finished) == [0, 1] and pool.num_free() == 5 and steps


def _swap_trace(seed):
    # with swapping nothing is recomputed: over the whole run each request's
    # chunks cover its prompt and all but its last output token exactly once,
    # in order; a swapped-out request keeps its progress and resumes with
    # ceil(computed/16) fresh blocks
    rng = np.random.default_rng(50 + seed)
    n = int(rng.integers(20, 80))
    pool = BlockPoolModel(n, 16, rng.permutation(n))
    budget = int(rng.integers(8, 200))
    s = SchedulerModel(pool, token_budget=budget, max_running=int(rng.integers(1, 12)), swap=True)
    rid, nxt = 0, {}
    swaps = 0
    for step in range(100000):
        if step < 200:
            for _ in range(int(rng.integers(0, 3))):
                prompt = int(rng.integers(1, 16 * max(1, n // 4)))
                s.add_request(rid, prompt=prompt, out=int(rng.integers(1, 30)))
                rid += 1
        before = {r: list(t) for r, t in pool.tables.items()}
        p = s.schedule()
        for r_, blocks, ln in p.swap_out:
            assert blocks == before[r_] and ln == s.reqs[r_].computed > 0
            swaps += 1
        for r_, blocks, ln in p.swap_in:
            assert len(blocks) == -(-ln // 16) and ln == s.reqs[r_].computed
        for r_, start, k, _ in p.items:
            assert start == nxt.get(r_, 0)       # contiguous, never repeated
            nxt[r_] = start + k
        s.commit()
        pool.check()
        if step >= 200 and not (s.waiting or s.running or s.swapped):
            break
    assert sorted(s.finished) == list(range(rid)) and pool.num_free() == n
    for r in s.reqs.values():
        assert nxt[r.rid] == r.prompt + r.out - 1
    return swaps


@pytest.mark.parametrize("seed", range(5))
def test_swap_mode_computes_every_token_exactly_once(seed):
    _swap_trace(seed)


def test_swap_traces_do_swap():
    # the traces are tight enough to exercise swapping
    assert sum(_swap_trace(k) for k in range(5)) > 10


def test_request_larger_than_the_pool_is_refused():
    s = SchedulerModel(BlockPoolModel(4), token_budget=64, max_running=4)
    s.add_request(0, prompt=60, out=5)           # 64 tokens = 4 blocks: fits
    with pytest.raises(ValueError):
        s.add_request(1, prompt=60, out=6)       # 65 tokens
