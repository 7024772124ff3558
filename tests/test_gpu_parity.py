"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Cache writes and tables are compared bit for bit; attention outputs element by
element within |gpu - oracle| <= 2e-3 + 1e-2 * |oracle| (fp16 inputs, fp32
accumulation, fp16 output).  Every pool byte starts as a NaN pattern, so an
unmasked read of an unwritten slot fails these tests."""
import numpy as np
import pytest
import torch

from gpu_util import (ATOL, FILL, RTOL, assert_close, assert_pools_bit_exact, gpu_run, log,
                      oracle_run, pools_to_logical, shared_oracle, shared_reference,
                      shared_workload)
from oracle import decode_attention_one, decode_reference, prefill_reference
from synth import make_mixed_workload, make_tiny_workload, make_workload
from synth.workloads import Workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------ the 5 configs

@pytest.mark.parametrize("cfg", ["1", "2", "4", "4b"])
def test_config_cache_and_decode(cfg):
    w = make_workload(cfg)
    st = oracle_run(w)
    res = gpu_run(w)
    assert res["step_slots"].tolist() == st.step_slots.tolist()
    assert [tuple(c) for c in res["step_copies"].tolist()] == st.step_copies
    n = assert_pools_bit_exact(res["cache"], st)
    err = assert_close(res["decode"], decode_reference(w, st), f"config {cfg} decode")
    log(f"config {cfg}: {n} live slots bit-exact, decode max err {err:.2e}")
    if cfg == "4":
        assert len(st.step_copies) == 0
    if cfg == "4b":
        assert len(st.step_copies) == w.batch - 1


def test_config3_full_size_decode():
    """The decode workload the benchmark times (split-K 512 + merge, work-list
    form), every output element against the oracle; the grid form and a
    second launch must give bitwise the same result."""
    w = shared_workload(3)
    st = shared_oracle(3)
    res = gpu_run(w, partition=512)
    n = assert_pools_bit_exact(res["cache"], st)
    err = assert_close(res["decode"], shared_reference(3, "decode"), "config 3 decode")
    log(f"config 3: {n} live slots bit-exact, decode max err {err:.2e}")
    from pagedattention_block_paged_reshape_amd.cache import DecodePlan
    grid = DecodePlan(res["cache"], w.decode_ids, w.n_q, w.scale, 512, worklist=False)
    g_out = grid.run(res["q"]).clone()
    again = res["plan"].run(res["q"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(g_out.view(torch.int16), res["decode"].view(torch.int16))
    assert torch.equal(again.view(torch.int16), res["decode"].view(torch.int16))


def test_config5_mixed_step():
    """8 decode requests at 32,768 tokens (64 partitions each) and the
    512-token prefill chunk at offset 49,488 over one pool, as two launches;
    every element of both outputs against the oracle."""
    w = shared_workload(5)
    st = shared_oracle(5)
    res = gpu_run(w, partition=512)
    assert_pools_bit_exact(res["cache"], st)
    err = assert_close(res["decode"], shared_reference(5, "decode"), "config 5 decode")
    errp = assert_close(res["prefill"], shared_reference(5, "prefill"),
                        "config 5 prefill (all 512 rows x 32 heads)")
    log(f"config 5: decode max err {err:.2e}, prefill max err {errp:.2e}")


# ---------------------------------------------------------- decode edges

RAGGED = [1, 2, 15, 16, 17, 31, 32, 33, 127, 511, 512, 513, 1000, 1537, 2049]


@pytest.mark.parametrize("worklist", [True, False])
@pytest.mark.parametrize("partition", [16, 32, 48, 256, 512, 4096])
def test_decode_partition_sizes(partition, worklist):
    w = make_tiny_workload(RAGGED, n_q=32, n_kv=8, d=128, seed=21, dist="normal")
    st = oracle_run(w)
    res = gpu_run(w, partition=partition, worklist=worklist)
    assert_close(res["decode"], decode_reference(w, st), f"partition {partition}")


@pytest.mark.parametrize("n_q,n_kv,d", [(16, 1, 128), (8, 8, 64), (4, 2, 64), (64, 8, 128),
                                        (12, 4, 128), (2, 2, 128), (16, 4, 64)])
def test_decode_head_shapes(n_q, n_kv, d):
    w = make_tiny_workload([1, 17, 64, 300, 700], n_q=n_q, n_kv=n_kv, d=d, seed=n_q * 7 + d,
                           dist="normal")
    st = oracle_run(w)
    res = gpu_run(w, partition=256)
    assert_close(res["decode"], decode_reference(w, st), f"heads {n_q}/{n_kv} d{d}")


def test_decode_single_token_returns_its_value_exactly():
    w = make_tiny_workload([1, 1, 1], n_q=16, n_kv=2, d=128, seed=5, dist="normal")
    st = oracle_run(w)
    res = gpu_run(w)
    out = res["decode"].cpu().numpy().view(np.uint16)
    for i in range(3):
        for h in range(16):
            assert np.array_equal(out[i, h], w.step_v[i, h // 8].view(np.uint16))


def test_decode_deterministic_and_placement_invariant():
    w = make_tiny_workload(RAGGED, n_q=32, n_kv=8, d=128, seed=33, dist="normal")
    a = gpu_run(w)
    again = a["plan"].run(a["q"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(a["decode"].view(torch.int16), again.view(torch.int16))
    for s in range(2):
        w.free_order = np.random.default_rng(500 + s).permutation(w.num_blocks).astype(np.int32)
        b = gpu_run(w)
        assert torch.equal(a["decode"].view(torch.int16), b["decode"].view(torch.int16))


def test_shared_prefix_equals_private_copies_bitwise():
    import pagedattention_block_paged_reshape_amd as pa
    shared = make_workload("4b")
    B = 16
    shared.decode_ids = shared.decode_ids[:B]
    shared.step_ids = shared.step_ids[:B]
    shared.step_n_new = shared.step_n_new[:B]
    shared.step_k, shared.step_v, shared.q = shared.step_k[:B], shared.step_v[:B], shared.q[:B]
    shared.setup = [op for op in shared.setup if op[0] != "fork" or op[2] < B]
    P = shared.notes["prefix"]
    private = Workload(
        name="private-copies", n_q=shared.n_q, n_kv=shared.n_kv, d=shared.d,
        scale=shared.scale, num_blocks=B * 70,
        free_order=np.random.default_rng(1).permutation(B * 70).astype(np.int32),
        setup=[("add", i) for i in range(B)] + [("append", list(range(B)), [P] * B)],
        setup_k=np.concatenate([shared.setup_k[:P]] * B),
        setup_v=np.concatenate([shared.setup_v[:P]] * B),
        step_ids=shared.step_ids, step_n_new=shared.step_n_new, step_k=shared.step_k,
        step_v=shared.step_v, decode_ids=shared.decode_ids, q=shared.q)
    a = gpu_run(shared)
    b = gpu_run(private)
    assert len(a["step_copies"]) == B - 1 and len(b["step_copies"]) == 0
    assert torch.equal(a["decode"].view(torch.int16), b["decode"].view(torch.int16))
    # the shared pool decodes with cached K/V loads, the private one streams
    # them; the load policy must not change a bit
    assert a["plan"].flags == pa.PA_DECODE_KEEP_KV and b["plan"].flags == 0
    a["plan"].flags = 0
    streamed = a["plan"].run(a["q"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(streamed.view(torch.int16), a["decode"].view(torch.int16))
    st = oracle_run(shared)
    assert_pools_bit_exact(a["cache"], st)
    assert_close(a["decode"], decode_reference(shared, st), "shared prefix")


@pytest.mark.parametrize("worklist", [True, False])
def test_decode_bad_table_entry_and_empty_request(worklist):
    import pagedattention_block_paged_reshape_amd as pa
    w = make_tiny_workload([40, 40, 40], n_q=8, n_kv=2, d=128, seed=8, dist="normal")
    st = oracle_run(w)
    res = gpu_run(w, worklist=worklist)
    plan = res["plan"]
    if worklist:   # the work list must cover the empty request too
        items = pa.pa_decode_work_items([40, 40, 0], 512)
        plan.items = torch.from_numpy(items.copy()).to("cuda:0")
        plan.n_items = len(items)
    good = res["decode"].clone()
    plan.tables[1, 1] = w.num_blocks + 7          # out of range: request 1 must read NaN
    plan.lens[2] = 0                              # empty request: zeros
    out = plan.run(res["q"]).clone()
    torch.cuda.synchronize()
    assert torch.isnan(out[1].float()).all()
    assert (out[2].float() == 0).all()
    assert torch.equal(out[0].view(torch.int16), good[0].view(torch.int16))
    assert_close(out[0:1], decode_reference(w, st)[0:1], "request next to a bad one")
    # host-side validation rejects bad geometry before any launch
    for n_q, part in ((7, 512), (8, 24), (8, 8192)):
        with pytest.raises(pa.PaError):
            pa.pa_paged_attention_decode(out, res["q"], plan.cache.kv, plan.tables,
                                         plan.max_blocks, plan.lens, 3, n_q, 0.1, part,
                                         plan.max_len, plan.items, plan.n_items, plan.workspace,
                                         plan.ws_bytes)


def test_reshape_and_cache_skips_negative_and_out_of_range_slots():
    import pagedattention_block_paged_reshape_amd as pa
    from pagedattention_block_paged_reshape_amd.cache import PagedKVCache
    cache = PagedKVCache(4, 2, 64, device="cuda:0", fill_byte=FILL)
    k = torch.randn(3, 2, 64, device="cuda:0").half()
    v = torch.randn(3, 2, 64, device="cuda:0").half()
    slots = torch.tensor([5, -1, 4 * 16 + 3], dtype=torch.int32, device="cuda:0")
    pa.pa_reshape_and_cache(k, v, slots, 3, cache.kv)
    torch.cuda.synchronize()
    kl, vl = pools_to_logical(cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy(), 64)
    assert np.array_equal(kl[0, :, 5, :], k[0].cpu().numpy())
    assert np.array_equal(vl[0, :, 5, :], v[0].cpu().numpy())
    written = np.zeros((4, 16), dtype=bool)
    written[0, 5] = True
    pattern = np.uint16(FILL | (FILL << 8))
    for pool in (kl, vl):
        rest = pool.view(np.uint16).transpose(0, 2, 1, 3)[~written]
        assert (rest == pattern).all()


# ---------------------------------------------------------------- prefill

@pytest.mark.parametrize("decode_lengths,q_start,chunk,n_q,n_kv,d", [
    ([], 0, 48, 4, 2, 128),            # whole causal prompt from position 0
    ([], 0, 200, 32, 8, 128),          # several query tiles, ragged tail
    ([17], 37, 100, 32, 8, 128),       # unaligned start, ragged
    ([5, 300], 1000, 300, 32, 8, 128),
    ([], 640, 129, 16, 16, 128),       # G = 1
    ([], 333, 77, 64, 8, 128),         # G = 8
    ([], 90, 50, 16, 1, 128),          # G = 16
    ([], 250, 130, 8, 2, 64),          # head_dim 64
    ([], 4093, 512, 32, 8, 128),       # several key splits
])
def test_prefill_chunk_parity(decode_lengths, q_start, chunk, n_q, n_kv, d):
    w = make_mixed_workload(decode_lengths, q_start, chunk, n_q=n_q, n_kv=n_kv, d=d,
                            seed=q_start + chunk)
    st = oracle_run(w)
    res = gpu_run(w)
    err = assert_close(res["prefill"], prefill_reference(w, st), "prefill chunk")
    if w.batch:
        assert_close(res["decode"], decode_reference(w, st), "decode in the mixed step")
    log(f"prefill q_start={q_start} chunk={chunk} G={n_q // n_kv} d={d}: max err {err:.2e}")


@pytest.mark.parametrize("q_start,chunk", [(700, 64), (2500, 300)])   # one split / several
def test_prefill_growing_scores_move_the_softmax_reference(q_start, chunk):
    """Key magnitudes grow with position (up to ~50x), so each row's scores
    climb far past what its softmax reference allows (a lane's sum of
    rounded P above 32,768) many times within one tile and split: every
    reference move rescales the partial sums, and the result must still be
    the oracle's softmax."""
    w = make_mixed_workload([], q_start, chunk, n_q=32, n_kv=8, d=128, seed=77 + chunk)
    ramp = lambda pos: (1.0 + pos / 50.0)[:, None, None]
    pos_setup = np.arange(len(w.setup_k), dtype=np.float64)
    pos_step = q_start + np.arange(len(w.step_k), dtype=np.float64)
    w.setup_k = (w.setup_k.astype(np.float64) * ramp(pos_setup)).astype(np.float16)
    w.step_k = (w.step_k.astype(np.float64) * ramp(pos_step)).astype(np.float16)
    st = oracle_run(w)
    res = gpu_run(w, decode=False)
    err = assert_close(res["prefill"], prefill_reference(w, st), "prefill, growing scores")
    log(f"prefill growing scores q_start={q_start} chunk={chunk}: max err {err:.2e}")


def test_prefill_last_row_matches_decode_kernel():
    """The chunk's last row sees exactly the prompt's keys, as a decode of
    the same request would."""
    w = make_mixed_workload([], 700, 64, n_q=32, n_kv=8, d=128, seed=2)
    res = gpu_run(w)
    from pagedattention_block_paged_reshape_amd.cache import DecodePlan
    plan = DecodePlan(res["cache"], [w.prefill.seq_id], w.n_q, w.scale, 512)
    dec = plan.run(res["qc"][-1:].contiguous()).clone()
    torch.cuda.synchronize()
    a = res["prefill"][-1].float().cpu().numpy()
    b = dec[0].float().cpu().numpy()
    assert np.allclose(a, b, rtol=RTOL, atol=ATOL)


@pytest.mark.parametrize("q_start,chunk", [(0, 40), (4093, 512)])   # one split / several
def test_prefill_bad_table_entry_reads_nan_and_empty_chunk_is_a_noop(q_start, chunk):
    """A table entry outside the pool makes the chunk's output NaN (no
    out-of-bounds read); a chunk of length 0 launches nothing and leaves the
    output untouched; bad geometry is rejected on the host."""
    import pagedattention_block_paged_reshape_amd as pa
    w = make_mixed_workload([], q_start, chunk, n_q=32, n_kv=8, d=128, seed=21)
    res = gpu_run(w, decode=False)
    pp, qc = res["pplan"], res["qc"]
    pp.table[0] = w.num_blocks + 3            # logical block 0: every row attends key 0
    out = pp.run(qc).clone()
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all()
    sentinel = torch.full_like(out, 7.0)
    pa.pa_paged_attention_prefill(sentinel, qc, pp.cache.kv, pp.table, pp.table_len, pp.q_start,
                                  0, pp.n_q, pp.scale, pp.workspace, pp.ws_bytes)
    torch.cuda.synchronize()
    assert (sentinel.float() == 7.0).all()
    for n_q, q0, c in ((30, pp.q_start, pp.chunk_len),                 # 30 % 8 != 0
                       (pp.n_q, pp.q_start, pp.table_len * 16 + 1),    # past the table
                       (pp.n_q, -1, pp.chunk_len)):
        with pytest.raises(pa.PaError):
            pa.pa_paged_attention_prefill(out, qc, pp.cache.kv, pp.table, pp.table_len, q0, c,
                                          n_q, pp.scale, pp.workspace, pp.ws_bytes)


@pytest.mark.parametrize("kv_dtype", ["fp16", "fp8"])
def test_swap_out_and_in_restores_kv_bitwise(kv_dtype):
    """A request swapped out to host memory, its blocks overwritten by another
    request, then swapped back in (into whatever blocks the free list gives):
    its K/V tiles come back bit for bit and the whole batch's decode output is
    bitwise unchanged."""
    import pagedattention_block_paged_reshape_amd as pa
    from pagedattention_block_paged_reshape_amd.cache import DecodePlan
    w = make_tiny_workload([33, 100, 517, 1200], n_q=8, n_kv=2, d=128, seed=9, dist="normal",
                           num_blocks=160)
    scales = dict(k_scale=0.02, v_scale=0.03) if kv_dtype == "fp8" else {}
    res = gpu_run(w, kv_dtype=kv_dtype, **scales)
    cache, out0 = res["cache"], res["decode"]
    victim = int(w.decode_ids[2])
    old_table, old_len = pa.pa_seq_table(cache.pool, victim)
    idx = torch.from_numpy(old_table.astype(np.int64)).to(cache.device)
    k_before = cache.k_pool[idx].clone()
    v_before = cache.v_pool[idx].clone()
    saved = cache.swap_out(victim)
    saved["event"].synchronize()
    assert saved["n"] == len(old_table) and saved["len"] == old_len
    # another request takes every free block (the victim's first) and writes them
    filler = 10 ** 6
    cache.add(filler)
    n_fill = pa.pa_num_free_blocks(cache.pool) * 16
    g = torch.Generator(device=cache.device).manual_seed(5)
    rows = lambda: torch.randn((n_fill, w.n_kv, w.d), generator=g, device=cache.device).half()
    cache.append([filler], [n_fill], rows(), rows())
    torch.cuda.synchronize()
    assert not torch.equal(cache.k_pool[idx].view(torch.uint8), k_before.view(torch.uint8))
    cache.free(filler)
    new_table = cache.swap_in(victim, saved)
    torch.cuda.synchronize()
    pa.pa_pool_check(cache.pool)
    assert pa.pa_seq_table(cache.pool, victim)[1] == old_len
    nidx = torch.from_numpy(np.asarray(new_table, dtype=np.int64)).to(cache.device)
    assert torch.equal(cache.k_pool[nidx].view(torch.uint8), k_before.view(torch.uint8))
    assert torch.equal(cache.v_pool[nidx].view(torch.uint8), v_before.view(torch.uint8))
    plan = DecodePlan(cache, w.decode_ids, w.n_q, w.scale, 512)
    out1 = plan.run(res["q"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out0.view(torch.int16))
    log(f"swap {kv_dtype}: {saved['n']} blocks out and back, old {old_table.tolist()[:4]}..., "
        f"new {list(new_table)[:4]}...")


def test_decode_empty_batch_is_a_noop():
    import pagedattention_block_paged_reshape_amd as pa
    w = make_tiny_workload([20], n_q=8, n_kv=2, d=128, seed=5, dist="normal")
    res = gpu_run(w)
    plan = res["plan"]
    sentinel = torch.full_like(res["decode"], 3.0)
    pa.pa_paged_attention_decode(sentinel, res["q"], plan.cache.kv, plan.tables, plan.max_blocks,
                                 plan.lens, 0, w.n_q, plan.scale, 512, plan.max_len, None, 0,
                                 plan.workspace, plan.ws_bytes)
    torch.cuda.synchronize()
    assert (sentinel.float() == 3.0).all()


@pytest.mark.parametrize("worklist_extra", ["other requests", "other partitions"])
def test_decode_work_list_entries_outside_the_batch_are_skipped(worklist_extra):
    """A work list built for other lengths (two requests the batch does not
    have, or longer requests with partitions the batch lacks) runs its extra
    entries as empty units: the outputs are bitwise those of the batch's own
    list, and no row outside the batch is written."""
    import pagedattention_block_paged_reshape_amd as pa
    w = make_tiny_workload([40, 700, 1300], n_q=16, n_kv=4, d=128, seed=61, dist="normal")
    res = gpu_run(w, partition=256)
    plan, good = res["plan"], res["decode"]
    lens = plan.lens.cpu().numpy().tolist()
    other = lens + [3000, 2500] if worklist_extra == "other requests" else [x + 900 for x in lens]
    items = pa.pa_decode_work_items(other, 256)
    assert len(items) > plan.n_items
    plan.items = torch.from_numpy(items.copy()).to("cuda:0")
    plan.n_items = len(items)
    # the output has room for two more requests, which must stay untouched
    big = torch.full((w.batch + 2, w.n_q, w.d), 5.0, dtype=torch.float16, device="cuda:0")
    plan.out = big[:w.batch]
    plan.run(res["q"])
    torch.cuda.synchronize()
    assert torch.equal(big[:w.batch].view(torch.int16), good.view(torch.int16))
    assert (big[w.batch:].float() == 5.0).all()


@pytest.mark.parametrize("case", ["config 2", "ragged, partition 32"])
def test_decode_worklist_give_up_writes_nan_not_stale_rows(case, monkeypatch):
    """The work-list kernel's LDS slot wait is bounded.  With the bound
    forced to 0 rounds from the host (a test hook; every wait still ends),
    a wavefront that finds a slot still busy gives up and the rest of its
    workgroup's units must come out NaN: every output row is either NaN or
    bitwise the normal run's, and the launch completes."""
    from pagedattention_block_paged_reshape_amd.cache import DecodePlan
    if case == "config 2":
        w, part = make_workload(2), 512
    else:
        w, part = make_tiny_workload(RAGGED * 3, n_q=32, n_kv=8, d=128, seed=71,
                                     dist="normal"), 32
    res = gpu_run(w, partition=part)
    good = res["decode"].float().cpu().numpy()
    plan = DecodePlan(res["cache"], w.decode_ids, w.n_q, w.scale, part)
    plan.out.fill_(3.0)                     # stale contents the give-up must not leave
    plan.workspace.fill_(0)
    monkeypatch.setenv("PA_DECODE_SPIN_LIMIT", "0")
    nan_rows = 0
    for rep in range(5):
        out = plan.run(res["q"]).clone()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        is_nan = np.isnan(got).all(axis=-1)
        same = (got.view(np.uint32) == good.view(np.uint32)).all(axis=-1)
        assert (is_nan | same).all(), f"{case}: a row is neither NaN nor the normal result"
        nan_rows += int(is_nan.sum())
    monkeypatch.delenv("PA_DECODE_SPIN_LIMIT")
    again = plan.run(res["q"]).clone()
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), res["decode"].view(torch.int16))
    log(f"give-up ({case}): {nan_rows} of {5 * good.shape[0] * good.shape[1]} rows NaN over 5 runs")
