"""GPU end to end for prefix caching (ngrok summary, "prefix caching":
requests that begin with the same tokens at the same positions share the
KV blocks of that prefix; one differing token ends the sharing; a block is
known by a hash of the previous block's hash and its own tokens).

A program of add_cached / append / register / free calls runs on the
library (pa_seq_add_cached, pa_seq_register, reshape_and_cache into a device
pool) and on the oracle's PrefixCachingPoolModel with its own pool model.
It makes a full-prefix hit, a partial hit, a hit that one differing token
cuts short, a hit that revives evictable blocks, and a miss on a prefix
whose first block was evicted.  Then every live request appends one token
and decode attends over the shared blocks:
  * tables, lengths, slots, copy lists, free and evictable lists equal the
    model's exactly; the pool equals the model's pool bit for bit;
  * decode (and a prefill chunk over a cached prefix) is within tolerance of
    the fp64 oracle element by element;
  * both are bitwise equal to the same requests held in private blocks with
    the same bytes (no sharing), and to a decode with streaming K/V loads.

K/V rows are a fixed function of (position, token id), so two requests with
the same tokens at the same positions have the same rows, as a model would
compute them."""
import numpy as np
import pytest
import torch

from gpu_util import FILL, assert_close, log, pools_to_logical
from oracle import PoolModel, PrefixCachingPoolModel, decode_attention_one
from oracle.attention import prefill_chunk_attention

pytestmark = pytest.mark.gpu

N_Q, N_KV, D = 32, 8, 128
SCALE = 1.0 / np.sqrt(D)
NUM_BLOCKS = 40


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def token_rows(positions, tokens):
    """fp16 K and V rows [n][N_KV][D] for tokens at positions: N(0,1) draws
    seeded by (position, token), so equal (position, token) pairs get equal
    rows."""
    k = np.empty((len(tokens), N_KV, D), dtype=np.float16)
    v = np.empty_like(k)
    for i, (p, t) in enumerate(zip(positions, tokens)):
        rng = np.random.default_rng((int(p) * 1_000_003 + int(t)) & 0x7FFFFFFF)
        k[i] = rng.standard_normal((N_KV, D), dtype=np.float32).astype(np.float16)
        v[i] = rng.standard_normal((N_KV, D), dtype=np.float32).astype(np.float16)
    return k, v


class Both:
    """The library (PagedKVCache) and the oracle (PrefixCachingPoolModel +
    PoolModel) driven by the same calls, compared after each one."""

    def __init__(self, free_order):
        from pagedattention_block_paged_reshape_amd.cache import PagedKVCache
        self.cache = PagedKVCache(NUM_BLOCKS, N_KV, D, free_order, "cuda:0", fill_byte=FILL)
        self.model = PrefixCachingPoolModel(NUM_BLOCKS, 16, free_order)
        self.pool = PoolModel(NUM_BLOCKS, N_KV, D)
        self.tokens = {}    # sequence -> its token ids so far

    def add_cached(self, sid, prompt):
        import pagedattention_block_paged_reshape_amd as pa
        got = pa.pa_seq_add_cached(self.cache.pool, sid, np.asarray(prompt, dtype=np.int32))
        want = self.model.add_cached(sid, prompt)
        assert got == want, (sid, got, want)
        self.tokens[sid] = list(prompt)
        return got

    def append(self, sid, n):
        """Append the sequence's next n tokens (its prompt's, then new ids)."""
        start = self.model.lens[sid]
        toks = self.tokens[sid]
        while len(toks) < start + n:
            toks.append(9000 + 37 * len(toks) + sid)
        k, v = token_rows(range(start, start + n), toks[start:start + n])
        slots, copies = self.cache.append([sid], [n], torch.from_numpy(k).to("cuda:0"),
                                          torch.from_numpy(v).to("cuda:0"))
        m_slots, m_copies = self.model.append([sid], [n])
        assert slots.tolist() == m_slots
        assert [tuple(c) for c in copies.tolist()] == m_copies
        self.pool.copy(m_copies)
        self.pool.write(k, v, m_slots)

    def register(self, sid, n_tokens):
        import pagedattention_block_paged_reshape_amd as pa
        toks = np.asarray(self.tokens[sid][:n_tokens], dtype=np.int32)
        got = pa.pa_seq_register(self.cache.pool, sid, toks)
        assert got == self.model.register(sid, toks.tolist())
        return got

    def free(self, sid):
        self.cache.free(sid)
        self.model.free_seq(sid)

    def check_host(self):
        import pagedattention_block_paged_reshape_amd as pa
        pa.pa_pool_check(self.cache.pool)
        self.model.check()
        for sid in self.model.tables:
            table, ln = pa.pa_seq_table(self.cache.pool, sid)
            assert table.tolist() == self.model.tables[sid] and ln == self.model.lens[sid], sid
        assert pa.pa_free_list(self.cache.pool).tolist() == self.model.free
        assert pa.pa_evictable_list(self.cache.pool).tolist() == self.model.evictable


def run_program():
    both = Both(np.random.default_rng(4242).permutation(NUM_BLOCKS).astype(np.int32))
    rng = np.random.default_rng(7)
    P = rng.integers(0, 32000, 80).tolist()           # shared system prompt, 5 blocks
    Q = rng.integers(0, 32000, 48).tolist()           # a prompt that goes evictable
    R = rng.integers(0, 32000, 32).tolist()           # a prompt whose first block is evicted
    A, B, C, Dq, E, F, H, FILLER, I = range(1, 10)
    hits = {}
    # A computes the prompt and publishes it
    hits[A] = both.add_cached(A, P)
    both.append(A, 80)
    assert both.register(A, 80) == 5
    # B: full-prefix hit, 20 more tokens
    hits[B] = both.add_cached(B, P + rng.integers(0, 32000, 20).tolist())
    both.append(B, 20)
    assert both.register(B, 96) == 1
    # C: the same tokens up to position 39, one differing token at 40
    c_prompt = P[:40] + [P[40] + 1] + P[41:60]
    hits[C] = both.add_cached(C, c_prompt)
    both.append(C, 60 - hits[C])
    # Dq: a shorter prompt, 3 full blocks of it are cached
    hits[Dq] = both.add_cached(Dq, P[:50])
    both.append(Dq, 50 - hits[Dq])
    # E publishes Q and finishes: its blocks become evictable
    hits[E] = both.add_cached(E, Q)
    both.append(E, 48)
    both.register(E, 48)
    both.free(E)
    evictable_q = list(both.model.evictable)
    # F reuses them (revived from the evictable list)
    hits[F] = both.add_cached(F, Q + [5, 6, 7, 8, 9])
    both.append(F, 5)
    both.free(A)
    # H publishes R and finishes; a filler request then takes every free block
    # and one more, which evicts R's first block (the oldest evictable)
    both.add_cached(H, R)
    both.append(H, 32)
    both.register(H, 32)
    both.free(H)
    evicted = both.model.evictable[0]
    both.add_cached(FILLER, [])
    both.append(FILLER, 16 * (len(both.model.free) + 1))
    assert evicted not in both.model.evictable
    both.free(FILLER)
    # I starts with R: its first block is gone, so nothing is shared
    hits[I] = both.add_cached(I, R + [1, 2, 3, 4])
    both.append(I, 36)
    both.check_host()
    assert hits == {A: 0, B: 80, C: 32, Dq: 48, E: 0, F: 48, I: 0}, hits
    assert all(b in both.model.tables[F] for b in evictable_q)
    live = [B, C, Dq, F, I]
    # the decode step: one new token per live request
    for sid in live:
        both.append(sid, 1)
    both.check_host()
    return both, live


def pool_bit_exact(both):
    """Valid slots of every block a request holds equal the model's pool."""
    kraw = both.cache.k_pool.cpu().numpy().view(np.uint16)
    vraw = both.cache.v_pool.cpu().numpy().view(np.uint16)
    kd, vd = pools_to_logical(kraw, vraw, D)
    n = 0
    for sid, table in both.model.tables.items():
        ln = both.model.lens[sid]
        for i, b in enumerate(table):
            c = min(16, ln - 16 * i)
            assert np.array_equal(kd[b, :, :c], both.pool.k[b, :, :c].view(np.uint16)), (sid, i)
            assert np.array_equal(vd[b, :, :c], both.pool.v[b, :, :c].view(np.uint16)), (sid, i)
            n += c
    return n


def private_copies(both, live):
    """The same requests, each in private blocks holding the same bytes."""
    from pagedattention_block_paged_reshape_amd.cache import PagedKVCache
    total = sum(-(-both.model.lens[s] // 16) for s in live)
    cache = PagedKVCache(total, N_KV, D, np.random.default_rng(3).permutation(total)
                         .astype(np.int32), "cuda:0", fill_byte=FILL)
    for sid in live:
        k, v = both.pool.gather(both.model.tables[sid], both.model.lens[sid])
        cache.add(sid)
        cache.append([sid], [len(k)], torch.from_numpy(k).to("cuda:0"),
                     torch.from_numpy(v).to("cuda:0"))
    return cache


def test_prefix_cache_decode_over_shared_blocks():
    import pagedattention_block_paged_reshape_amd as pa
    from pagedattention_block_paged_reshape_amd.cache import DecodePlan
    both, live = run_program()
    n = pool_bit_exact(both)
    stats = pa.pa_pool_get_stats(both.cache.pool)
    assert stats["num_shared"] > 0
    q = np.random.default_rng(11).standard_normal((len(live), N_Q, D),
                                                   dtype=np.float32).astype(np.float16)
    dq = torch.from_numpy(q).to("cuda:0")
    plan = DecodePlan(both.cache, live, N_Q, SCALE, 512)
    assert plan.flags == pa.PA_DECODE_KEEP_KV          # chosen from the pool stats
    out = plan.run(dq).clone()
    plan.flags = 0
    streamed = plan.run(dq).clone()
    priv = private_copies(both, live)
    pplan = DecodePlan(priv, live, N_Q, SCALE, 512)
    assert pplan.flags == 0
    out_priv = pplan.run(dq).clone()
    torch.cuda.synchronize()
    ref = np.stack([decode_attention_one(q[i], *both.pool.gather_values(
        both.model.tables[s], both.model.lens[s]), SCALE) for i, s in enumerate(live)])
    err = assert_close(out, ref, "decode over cached prefix blocks")
    assert torch.equal(out.view(torch.int16), streamed.view(torch.int16))
    assert torch.equal(out.view(torch.int16), out_priv.view(torch.int16))
    log(f"prefix cache decode: {n} live slots bit-exact, {stats['num_shared']} shared blocks, "
        f"lengths {[both.model.lens[s] for s in live]}, max err {err:.2e}")


def test_prefix_cache_prefill_chunk_over_cached_prefix():
    """Request B's own tokens (positions 80..100) as a causal chunk whose
    first 80 keys live in blocks it got from the cache."""
    from pagedattention_block_paged_reshape_amd.cache import PrefillPlan
    both, live = run_program()
    sid, q_start = live[0], 80
    ln = both.model.lens[sid]
    chunk = ln - q_start
    q = np.random.default_rng(12).standard_normal((chunk, N_Q, D),
                                                   dtype=np.float32).astype(np.float16)
    dq = torch.from_numpy(q).to("cuda:0")
    out = PrefillPlan(both.cache, sid, q_start, chunk, N_Q, SCALE).run(dq).clone()
    priv = private_copies(both, live)
    out_priv = PrefillPlan(priv, sid, q_start, chunk, N_Q, SCALE).run(dq).clone()
    torch.cuda.synchronize()
    k, v = both.pool.gather_values(both.model.tables[sid], ln)
    ref = prefill_chunk_attention(q, k, v, q_start, SCALE)
    err = assert_close(out, ref, "prefill chunk over cached prefix blocks")
    assert torch.equal(out.view(torch.int16), out_priv.view(torch.int16))
    log(f"prefix cache prefill: rows {q_start}..{ln - 1}, max err {err:.2e}")
