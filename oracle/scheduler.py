"""Oracle model of the continuous-batching scheduler around the paged cache.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What it follows:
  * ngrok summary, scheduler section: every forward pass the scheduler picks
    the tokens of the batch within a token budget, requests that are already
    running (decoding) first, then waiting requests' prefill while budget is
    left; a very long prompt is split into chunks that fit the budget
    (chunked prefill); when KV blocks run out, the request added most
    recently is preempted: its blocks are freed, it goes back to the head of
    the waiting queue and its tokens are computed again later.
  * ta-paperlens, "scheduler skeleton": admit from the waiting queue while the
    head can be allocated; step every running request; drop finished ones and
    free their blocks; while out of blocks, preempt running[-1].

Readings (the pages leave these open):
  * A request is (prompt length, output length).  Its input is the prompt
    followed by its generated tokens; one step processes a chunk of its
    not-yet-computed input.  When a step computes the last input token, the
    request produces one new token (counted in ``generated``); it is done
    when generated == output length, and is then freed at the end of the
    step.
  * Order inside a step: running requests in admission order, those whose
    whole input but the newest token is computed (decode: 1 token) before
    those still in prefill (a chunk of min(remaining, budget left)); then
    waiting requests in queue order, each admitted only if the pool can hold
    the blocks of its first chunk and fewer than ``max_running`` run.  A
    running request that gets no budget simply waits (it keeps its blocks).
  * Block reservation is one append of all the step's chunks in that order.
    If it does not fit, the most recently admitted running request is
    preempted (freed, its computed count reset to 0, put at the head of the
    waiting queue, removed from this step) and the reservation retried;
    requests admitted in this very step count as running for this.
  * A preempted request recomputes prompt + generated tokens from position 0
    (recompute mode).
  * Swap mode (the skeleton's other choice: move the preempted request to CPU
    memory instead of dropping it): the victim keeps its computed count, its
    blocks' K/V are copied out and its blocks released (exactly as a free),
    and it goes to the head of a swapped queue.  At the start of each step,
    before anything else, swapped requests resume from the head of that
    queue while fewer than ``max_running`` run and the free blocks cover the
    request's ceil(computed/16) blocks plus one block per running request
    (headroom for their next tokens); a resumed request takes fresh blocks
    in logical order (as a new request appending ``computed`` tokens) and
    runs like any other.  A victim with nothing computed is preempted as in
    recompute mode; a victim resumed in the same step goes back to the head
    of the swapped queue with its fresh blocks released and no data moved
    (its saved copy is still the current one).
"""
from __future__ import annotations

from collections import deque
from dataclasses import dataclass, field
from typing import Deque, Dict, List, Tuple

from .allocator import BlockPoolModel, OutOfBlocks


@dataclass
class Req:
    rid: int
    prompt: int
    out: int
    computed: int = 0
    generated: int = 0
    preemptions: int = 0

    @property
    def total(self) -> int:
        return self.prompt + self.generated


@dataclass
class StepPlan:
    items: List[Tuple[int, int, int, int]] = field(default_factory=list)  # rid, start, n, decode
    slots: List[int] = field(default_factory=list)
    copies: List[Tuple[int, int, int]] = field(default_factory=list)
    preempted: List[int] = field(default_factory=list)
    admitted: List[int] = field(default_factory=list)
    # swap mode: (rid, blocks in logical order, computed length) moved out /
    # back in this step, in the order they happen
    swap_out: List[Tuple[int, List[int], int]] = field(default_factory=list)
    swap_in: List[Tuple[int, List[int], int]] = field(default_factory=list)


class SchedulerModel:
    def __init__(self, pool: BlockPoolModel, token_budget: int, max_running: int,
                 swap: bool = False):
        if token_budget < 1 or max_running < 1:
            raise ValueError("budget and max_running must be positive")
        self.pool = pool
        self.budget = int(token_budget)
        self.max_running = int(max_running)
        self.reqs: Dict[int, Req] = {}
        self.waiting: Deque[int] = deque()
        self.running: List[int] = []
        self.finished: List[int] = []
        self.last: StepPlan = StepPlan()
        self.swap = bool(swap)
        self.swapped: Deque[int] = deque()

    def add_request(self, rid: int, prompt: int, out: int) -> None:
        """A request that could not fit the pool even alone (its prompt and
        all but its last output token) is refused: it would be preempted
        forever."""
        if rid in self.reqs or prompt < 1 or out < 1:
            raise ValueError("bad request")
        if self._blocks_for_new(prompt + out - 1) > self.pool.num_blocks:
            raise ValueError("request larger than the pool")
        self.reqs[rid] = Req(rid, int(prompt), int(out))
        self.waiting.append(rid)

    def _blocks_for_new(self, n: int) -> int:
        return -(-n // self.pool.block_size)

    def schedule(self) -> StepPlan:
        """Plan one step: which chunks run, their slots, copies, preemptions."""
        plan = StepPlan()
        budget = self.budget
        chunks: List[Tuple[int, int]] = []      # (rid, n) in reservation order
        while self.swapped and len(self.running) < self.max_running:
            r = self.reqs[self.swapped[0]]
            if self._blocks_for_new(r.computed) + len(self.running) > self.pool.num_free():
                break
            self.swapped.popleft()
            self.pool.add(r.rid)
            self.pool.append([r.rid], [r.computed])
            self.running.append(r.rid)
            plan.swap_in.append((r.rid, list(self.pool.tables[r.rid]), r.computed))
        for rid in self.running:                 # decode first
            r = self.reqs[rid]
            if r.total - r.computed == 1 and r.computed >= r.prompt and budget > 0:
                chunks.append((rid, 1))
                budget -= 1
        for rid in self.running:                 # then prefill chunks of running requests
            r = self.reqs[rid]
            if not (r.total - r.computed == 1 and r.computed >= r.prompt) and budget > 0:
                n = min(r.total - r.computed, budget)
                chunks.append((rid, n))
                budget -= n
        free = self.pool.num_free()
        need_running = self.pool.blocks_needed([c[0] for c in chunks], [c[1] for c in chunks]) \
            if chunks else 0
        spare = free - need_running
        while self.waiting and budget > 0 and len(self.running) < self.max_running:
            r = self.reqs[self.waiting[0]]
            n = min(r.total - r.computed, budget)
            blocks = self._blocks_for_new(n)
            if blocks > spare:
                break
            self.waiting.popleft()
            self.pool.add(r.rid)
            self.running.append(r.rid)
            plan.admitted.append(r.rid)
            chunks.append((r.rid, n))
            budget -= n
            spare -= blocks
        while True:
            try:
                slots, copies = self.pool.append([c[0] for c in chunks], [c[1] for c in chunks])
                break
            except OutOfBlocks:
                victim = self.running.pop()
                v = self.reqs[victim]
                resumed = [i for i, x in enumerate(plan.swap_in) if x[0] == victim]
                if self.swap and resumed:
                    # back to where it was: its saved copy is still current
                    self.pool.free_seq(victim)
                    del plan.swap_in[resumed[0]]
                    self.swapped.appendleft(victim)
                elif self.swap and v.computed > 0:
                    plan.swap_out.append((victim, list(self.pool.tables[victim]), v.computed))
                    self.pool.free_seq(victim)
                    self.swapped.appendleft(victim)
                else:
                    self.pool.free_seq(victim)
                    v.computed = 0
                    self.waiting.appendleft(victim)
                v.preemptions += 1
                plan.preempted.append(victim)
                chunks = [c for c in chunks if c[0] != victim]
                if victim in plan.admitted:
                    plan.admitted.remove(victim)
        for rid, n in chunks:
            r = self.reqs[rid]
            decode = int(n == 1 and r.computed >= r.prompt)   # the newest token only
            plan.items.append((rid, r.computed, n, decode))
        plan.slots, plan.copies = slots, copies
        self.last = plan
        return plan

    def commit(self) -> List[int]:
        """The planned chunks were computed: advance, emit tokens, retire
        finished requests (their blocks are freed).  Returns the finished ids."""
        done = []
        for rid, start, n, _ in self.last.items:
            r = self.reqs[rid]
            r.computed = start + n
            if r.computed == r.total:
                r.generated += 1
                if r.generated == r.out:
                    done.append(rid)
        for rid in done:
            self.running.remove(rid)
            self.pool.free_seq(rid)
            self.finished.append(rid)
        self.last = StepPlan()
        return done
