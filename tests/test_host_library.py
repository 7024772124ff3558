"""The C-ABI library on the CPU: it loads, exports every symbol include/pa.h
declares, and its host block manager matches the oracle's allocator model
exactly (tables, slot mapping, copy-on-write lists, free list, errors).
No GPU work is launched here."""
import os
import re
import subprocess

import numpy as np
import pytest

import pagedattention_block_paged_reshape_amd as pa
from pagedattention_block_paged_reshape_amd import _lib
from oracle import BlockPoolModel, OutOfBlocks, kv_bytes_per_token
from synth import make_tiny_workload, make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 20
    nm = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\s[TW]\s+(\w+)$", nm, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    assert set(names) == set(_lib.EXPORTED)


def test_staging_helpers_reject_bad_arguments_before_any_device_call():
    import ctypes as C
    out = C.c_void_p()
    assert _lib.LIB.pa_host_device_pointer(None, C.byref(out)) == _lib.PA_ERR_INVALID
    assert _lib.LIB.pa_host_device_pointer(16, None) == _lib.PA_ERR_INVALID
    # null, misaligned, or not whole 16-byte chunks
    assert _lib.LIB.pa_stage_copy(None, 256, 16, None) == _lib.PA_ERR_INVALID
    assert _lib.LIB.pa_stage_copy(256, None, 16, None) == _lib.PA_ERR_INVALID
    assert _lib.LIB.pa_stage_copy(256 + 4, 512, 16, None) == _lib.PA_ERR_INVALID
    assert _lib.LIB.pa_stage_copy(256, 512 + 8, 16, None) == _lib.PA_ERR_INVALID
    assert _lib.LIB.pa_stage_copy(256, 512, 20, None) == _lib.PA_ERR_INVALID
    # nothing to copy: no launch
    assert _lib.LIB.pa_stage_copy(256, 512, 0, None) == _lib.PA_OK
    # pa_stage_update: the copy's rules, plus the update list's
    up = _lib.LIB.pa_stage_update
    assert up(None, 512, 16, 1024, 1, 2048, 8, None) == _lib.PA_ERR_INVALID
    assert up(256 + 4, 512, 16, 1024, 1, 2048, 8, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 20, 1024, 1, 2048, 8, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 16, None, 1, 2048, 8, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 16, 1024, 1, None, 8, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 16, 1024 + 4, 1, 2048, 8, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 16, 1024, 1, 2048 + 2, 8, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 16, 1024, -1, 2048, 8, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 16, 1024, 1, 2048, -1, None) == _lib.PA_ERR_INVALID
    assert up(256, 512, 16, 1024, 1, 2048, 1 << 31, None) == _lib.PA_ERR_INVALID
    # nothing to copy and no updates: no launch (null pointers allowed then)
    assert up(None, None, 0, None, 0, None, 0, None) == _lib.PA_OK


def test_status_strings_and_kv_bytes():
    assert pa.status_string(0) == "ok"
    assert "out of blocks" in pa.status_string(2)
    assert pa.pa_kv_bytes_per_token(32, 8, 128, 2) == kv_bytes_per_token(32, 8, 128, 2) == 131072


def test_pool_create_rejects_bad_geometry():
    with pytest.raises(pa.PaError):
        pa.pa_pool_create(0)
    with pytest.raises(pa.PaError):
        pa.pa_pool_create(8, block_size=32)
    with pytest.raises(pa.PaError):
        pa.pa_pool_create(4, free_order=[0, 1, 1, 3])
    with pytest.raises(pa.PaError):
        pa.pa_pool_create(1 << 27)  # 2^27 * 16 slots overflows int32


class Twin:
    """Library pool and oracle model driven by the same operations."""

    def __init__(self, n, order=None):
        self.lib = pa.pa_pool_create(n, order)
        self.ref = BlockPoolModel(n, 16, order)

    def close(self):
        pa.pa_pool_destroy(self.lib)

    def compare(self):
        pa.pa_pool_check(self.lib)
        self.ref.check()
        assert pa.pa_free_list(self.lib).tolist() == self.ref.free
        for s in self.ref.tables:
            t, ln = pa.pa_seq_table(self.lib, s)
            assert t.tolist() == self.ref.tables[s] and ln == self.ref.lens[s]
        for b in range(self.ref.num_blocks):
            assert pa.pa_ref_count(self.lib, b) == self.ref.ref[b]


@pytest.mark.parametrize("seed", range(8))
def test_random_programs_match_oracle_exactly(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(4, 40))
    tw = Twin(n, rng.permutation(n))
    live, nid = [], 0
    try:
        for _ in range(150):
            op = int(rng.integers(0, 7))
            if op == 0 or not live:
                pa.pa_seq_add(tw.lib, nid)
                tw.ref.add(nid)
                live.append(nid)
                nid += 1
            elif op == 1:
                p = int(rng.choice(live))
                pa.pa_seq_fork(tw.lib, p, nid)
                tw.ref.fork(p, nid)
                live.append(nid)
                nid += 1
            elif op == 2 and len(live) > 1:
                s = int(rng.choice(live))
                pa.pa_seq_free(tw.lib, s)
                tw.ref.free_seq(s)
                live.remove(s)
            else:
                k = int(rng.integers(1, min(5, len(live)) + 1))
                ids = [int(x) for x in rng.choice(live, size=k, replace=False)]
                nn = [int(x) for x in rng.integers(0, 35, size=k)]
                need_ref = None
                need_ref = tw.ref.blocks_needed(ids, nn)
                assert pa.pa_can_append(tw.lib, ids, nn) == need_ref
                try:
                    exp = tw.ref.append(ids, nn)
                except OutOfBlocks:
                    with pytest.raises(pa.OutOfBlocksError):
                        pa.pa_append_slots(tw.lib, ids, nn)
                else:
                    slots, copies = pa.pa_append_slots(tw.lib, ids, nn)
                    assert slots.tolist() == exp[0]
                    assert [tuple(c) for c in copies.tolist()] == exp[1]
            tw.compare()
            st = pa.pa_pool_get_stats(tw.lib)
            assert st["num_shared"] == sum(1 for r in tw.ref.ref if r > 1)
        st = pa.pa_pool_get_stats(tw.lib)
        assert st["num_free"] == len(tw.ref.free) and st["num_seqs"] == len(live)
    finally:
        tw.close()


@pytest.mark.parametrize("seed", range(6))
def test_swap_out_and_in_match_free_and_reallocation_in_the_oracle(seed):
    """Swapping a sequence out releases its blocks exactly as freeing it does
    (same free list, same reference counts, shared blocks kept by their other
    holders); swapping it back in takes ceil(len/16) fresh blocks in logical
    order, as a new sequence appending len tokens does in the oracle's model,
    and fails with no state change when the pool is short."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(6, 40))
    tw = Twin(n, rng.permutation(n))
    live, swapped, nid = [], {}, 0
    try:
        for _ in range(200):
            op = int(rng.integers(0, 8))
            if op == 0 or not live:
                pa.pa_seq_add(tw.lib, nid)
                tw.ref.add(nid)
                live.append(nid)
                nid += 1
            elif op == 1:
                p = int(rng.choice(live))
                pa.pa_seq_fork(tw.lib, p, nid)
                tw.ref.fork(p, nid)
                live.append(nid)
                nid += 1
            elif op in (2, 3) and len(live) > 1:
                s = int(rng.choice(live))
                exp_blocks, exp_len = list(tw.ref.tables[s]), tw.ref.lens[s]
                blocks, ln = pa.pa_seq_swap_out(tw.lib, s)
                assert blocks.tolist() == exp_blocks and ln == exp_len
                tw.ref.free_seq(s)
                live.remove(s)
                swapped[s] = ln
            elif op == 4 and swapped:
                s = int(rng.choice(list(swapped)))
                ln = swapped[s]
                need = -(-ln // 16)
                if need > len(tw.ref.free):
                    before = pa.pa_free_list(tw.lib).tolist()
                    with pytest.raises(pa.OutOfBlocksError):
                        pa.pa_seq_swap_in(tw.lib, s, ln)
                    assert pa.pa_free_list(tw.lib).tolist() == before
                else:
                    blocks = pa.pa_seq_swap_in(tw.lib, s, ln)
                    tw.ref.add(s)
                    if ln:
                        tw.ref.append([s], [ln])
                    assert blocks.tolist() == tw.ref.tables[s]
                    del swapped[s]
                    live.append(s)
            else:
                k = int(rng.integers(1, min(4, len(live)) + 1))
                ids = [int(x) for x in rng.choice(live, size=k, replace=False)]
                nn = [int(x) for x in rng.integers(0, 35, size=k)]
                try:
                    exp = tw.ref.append(ids, nn)
                except OutOfBlocks:
                    with pytest.raises(pa.OutOfBlocksError):
                        pa.pa_append_slots(tw.lib, ids, nn)
                else:
                    slots, copies = pa.pa_append_slots(tw.lib, ids, nn)
                    assert slots.tolist() == exp[0]
            tw.compare()
            pa.pa_pool_check(tw.lib)
        with pytest.raises(pa.PaError):             # swapped-out ids are unknown
            for s in swapped:
                pa.pa_seq_swap_out(tw.lib, s)
            raise pa.PaError(1, "no swapped sequence left to probe")
        if live:
            with pytest.raises(pa.PaError):         # a live id cannot be swapped in
                pa.pa_seq_swap_in(tw.lib, live[0], 16)
    finally:
        tw.close()


def test_errors_leave_state_unchanged():
    tw = Twin(3)
    try:
        pa.pa_seq_add(tw.lib, 0)
        tw.ref.add(0)
        with pytest.raises(pa.PaError) as e:
            pa.pa_seq_add(tw.lib, 0)
        assert e.value.status == _lib.PA_ERR_EXISTS
        with pytest.raises(pa.PaError) as e:
            pa.pa_seq_fork(tw.lib, 5, 6)
        assert e.value.status == _lib.PA_ERR_UNKNOWN_SEQ
        with pytest.raises(pa.PaError) as e:
            pa.pa_append_slots(tw.lib, [0, 0], [1, 1])       # duplicate id
        assert e.value.status == _lib.PA_ERR_INVALID
        with pytest.raises(pa.PaError):
            pa.pa_append_slots(tw.lib, [0], [-1])
        with pytest.raises(pa.OutOfBlocksError):
            pa.pa_append_slots(tw.lib, [0], [49])            # 4 blocks, 3 exist
        tw.compare()
        pa.pa_append_slots(tw.lib, [0], [48])
        tw.ref.append([0], [48])
        tw.compare()
        with pytest.raises(pa.PaError) as e:
            pa.pa_block_tables(tw.lib, [0], 2)               # table has 3 blocks
        assert e.value.status == _lib.PA_ERR_CAPACITY
    finally:
        tw.close()


def _program_on_library(w):
    pool = pa.pa_pool_create(w.num_blocks, w.free_order)
    slots_all, copies_all = [], []
    for op in w.setup:
        if op[0] == "add":
            pa.pa_seq_add(pool, op[1])
        elif op[0] == "fork":
            pa.pa_seq_fork(pool, op[1], op[2])
        else:
            s, c = pa.pa_append_slots(pool, op[1], op[2])
            slots_all.extend(s.tolist())
            copies_all.extend(map(tuple, c.tolist()))
    step_slots, step_copies = pa.pa_append_slots(pool, w.step_ids, w.step_n_new)
    return pool, slots_all, copies_all, step_slots.tolist(), [tuple(c) for c in step_copies]


@pytest.mark.parametrize("cfg", ["1", "4b"])
def test_workload_tables_match_oracle(cfg):
    w = make_workload(cfg)
    pool, s_setup, c_setup, s_step, c_step = _program_on_library(w)
    ref = BlockPoolModel(w.num_blocks, 16, w.free_order)
    exp_setup = []
    for op in w.setup:
        if op[0] == "add":
            ref.add(op[1])
        elif op[0] == "fork":
            ref.fork(op[1], op[2])
        else:
            exp_setup.extend(ref.append(op[1], op[2])[0])
    exp_step, exp_copies = ref.append(w.step_ids.tolist(), w.step_n_new.tolist())
    assert s_setup == exp_setup and s_step == exp_step and c_step == exp_copies
    ids = w.decode_ids.tolist()
    mb = max(len(ref.tables[i]) for i in ids)
    tab, lens = pa.pa_block_tables(pool, ids, mb + 3)
    rows, lens_ref = ref.block_tables(ids, mb + 3)
    assert tab.tolist() == rows and lens.tolist() == lens_ref
    if cfg == "4b":
        assert len(c_step) == w.batch - 1          # every sharer but the last copies
    pa.pa_pool_check(pool)
    pa.pa_pool_destroy(pool)


def test_ragged_workload_tables_match_oracle():
    w = make_tiny_workload([1, 2, 15, 16, 17, 31, 32, 33, 100, 257], n_q=8, n_kv=2, d=64,
                           seed=3)
    pool, s_setup, _, s_step, _ = _program_on_library(w)
    ref = BlockPoolModel(w.num_blocks, 16, w.free_order)
    for op in w.setup:
        if op[0] == "add":
            ref.add(op[1])
        else:
            assert ref.append(op[1], op[2])[0] == s_setup
    assert ref.append(w.step_ids.tolist(), w.step_n_new.tolist())[0] == s_step
    pa.pa_pool_destroy(pool)


@pytest.mark.parametrize("partition", [16, 48, 512, 4096])
def test_decode_work_items_cover_every_unit_largest_first(partition):
    rng = np.random.default_rng(partition)
    lens = rng.integers(0, 5000, size=97).tolist() + [0, 1, 16, 17, partition, partition + 1]
    items = pa.pa_decode_work_items(lens, partition)
    pb = partition // 16
    units = []
    for b, L in enumerate(lens):
        nb = -(-L // 16)
        if L == 0:
            units.append((b, 0, 0))
        for p in range(-(-nb // pb)):
            units.append((b, p, min(pb, nb - p * pb)))
    got = [(int(x) >> 16, int(x) & 0xFFFF) for x in items]
    assert sorted(got) == sorted((b, p) for b, p, _ in units)
    size = {(b, p): s for b, p, s in units}
    sizes = [size[u] for u in got]
    assert sizes == sorted(sizes, reverse=True)
    # ties keep (request, partition) order
    for i in range(1, len(got)):
        if sizes[i] == sizes[i - 1]:
            assert got[i] > got[i - 1]


def test_decode_work_items_errors():
    with pytest.raises(pa.PaError):
        pa.pa_decode_work_items([5, -1], 512)
    with pytest.raises(pa.PaError):
        pa.pa_decode_work_items([5], 24)


def test_tile_layout_converter_matches_the_header_formulas():
    """The tests read device pools through gpu_util.pools_to_logical; check it
    against the per-element offsets include/pa.h states for both tiles."""
    gpu_util = pytest.importorskip("gpu_util")
    for d in (64, 128):
        kraw = np.full((1, 1, 16 * d), -1, dtype=np.int32)
        vraw = np.full((1, 1, 16 * d), -1, dtype=np.int32)
        for s in range(16):
            for c in range(d):
                kraw[0, 0, (c // 8) * 128 + s * 8 + c % 8] = s * 1000 + c
                vraw[0, 0, (c // 32) * 512 + (s // 4) * 128 + (c % 16) * 8
                     + ((c // 16) % 2) * 4 + s % 4] = s * 1000 + c
        assert (kraw >= 0).all() and (vraw >= 0).all()      # both maps are onto
        k, v = gpu_util.pools_to_logical(kraw, vraw, d)
        want = np.arange(16)[:, None] * 1000 + np.arange(d)[None, :]
        assert np.array_equal(k[0, 0], want) and np.array_equal(v[0, 0], want)


def test_fp8_tile_layout_converter_matches_the_header_formulas():
    gpu_util = pytest.importorskip("gpu_util")
    for d in (64, 128):
        kraw = np.full((1, 1, 16 * d), -1, dtype=np.int32)
        vraw = np.full((1, 1, 16 * d), -1, dtype=np.int32)
        for s in range(16):
            for c in range(d):
                kraw[0, 0, (c // 64) * 1024 + ((c // 8) % 4) * 256 + s * 16 + ((c // 32) % 2) * 8
                     + c % 8] = s * 1000 + c
                vraw[0, 0, (c // 64) * 1024 + (s // 4) * 256 + (c % 16) * 16 + ((c // 32) % 2) * 8
                     + ((c // 16) % 2) * 4 + s % 4] = s * 1000 + c
        assert (kraw >= 0).all() and (vraw >= 0).all()
        k, v = gpu_util.pools8_to_logical(kraw, vraw, d)
        want = np.arange(16)[:, None] * 1000 + np.arange(d)[None, :]
        assert np.array_equal(k[0, 0], want) and np.array_equal(v[0, 0], want)


def test_fp8_calls_reject_bad_scales_before_any_launch():
    # dummy addresses, never dereferenced: every call below fails or returns
    # on the host
    for ks, vs in ((0.0, 1.0), (1.0, -2.0), (float("nan"), 1.0), (1.0, float("inf"))):
        kv = pa.kv_view_fp8(None, None, 4, 2, 64, ks, vs)
        kv.k_pool = kv.v_pool = 1 << 20
        with pytest.raises(pa.PaError):
            pa.pa_reshape_and_cache_fp8(1 << 21, 1 << 22, 1 << 23, 3, kv)
        with pytest.raises(pa.PaError):
            pa.pa_copy_blocks_fp8(1 << 21, 1, kv)
        with pytest.raises(pa.PaError):
            pa.pa_paged_attention_decode_fp8(1 << 21, 1 << 22, kv, 1 << 23, 4, 1 << 24, 1, 4,
                                             0.125, 512, 64, None, 0, None, 0)
    kv = pa.kv_view_fp8(None, None, 4, 2, 64, 0.5, 2.0)
    kv.k_pool = kv.v_pool = 1 << 20
    pa.pa_reshape_and_cache_fp8(1 << 21, 1 << 22, 1 << 23, 0, kv)          # nothing to store
    with pytest.raises(pa.PaError):
        pa.pa_paged_attention_decode_fp8(1 << 21, 1 << 22, kv, 1 << 23, 4, 1 << 24, 0, 4,
                                         0.125, 512, 64, None, 0, None, 0, flags=4)
    pa.pa_paged_attention_decode_fp8(1 << 21, 1 << 22, kv, 1 << 23, 4, 1 << 24, 0, 4, 0.125,
                                     512, 64, None, 0, None, 0)               # batch 0


def test_decode_rejects_unknown_flags_before_any_launch():
    # argument checks run on the host before anything touches the GPU: the
    # dummy addresses below are never dereferenced
    kv = pa.kv_view(None, None, 4, 2, 64)
    kv.k_pool = kv.v_pool = 1 << 20
    args = dict(out=1 << 21, q=1 << 22, kv=kv, tables=1 << 23, max_blocks=4,
                seq_lens=1 << 24, batch=0, num_q_heads=4, scale=0.125, partition_size=512,
                max_seq_len=64, work_items=None, n_items=0, workspace=None, workspace_bytes=0)
    with pytest.raises(pa.PaError):
        pa.pa_paged_attention_decode(**args, flags=2)
    pa.pa_paged_attention_decode(**args, flags=pa.PA_DECODE_KEEP_KV)   # batch 0: nothing to do
    pa.pa_paged_attention_decode(**args, flags=0)


def test_attention_calls_reject_bad_scales_before_any_launch():
    """The softmax scale must be positive and finite for decode, prefill and
    the mixed launch (the kernels take max(c * s) = c * max(s)); the check
    comes before the early returns of empty calls.  Dummy addresses, never
    dereferenced."""
    kv = pa.kv_view(None, None, 64, 8, 128)
    kv.k_pool = kv.v_pool = 1 << 20
    dec = pa.decode_batch(1 << 21, 1 << 22, 1 << 23, 256, 1 << 24, 4, 512, 4096, 1 << 25, 32)
    pf = pa.prefill_chunk(1 << 26, 1 << 27, 1 << 28, 3125, 49488, 512)
    empty_dec = pa.decode_batch(1 << 21, 1 << 22, 1 << 23, 256, 1 << 24, 0, 512, 4096, None, 0)
    empty_pf = pa.prefill_chunk(1 << 26, 1 << 27, 1 << 28, 3125, 49488, 0)
    big = 1 << 40
    for scale in (0.0, -0.088, float("inf"), float("-inf"), float("nan")):
        for batch in (4, 0):
            with pytest.raises(pa.PaError):
                pa.pa_paged_attention_decode(1 << 21, 1 << 22, kv, 1 << 23, 256, 1 << 24, batch,
                                             32, scale, 512, 4096, 1 << 25, 32, 1 << 29, big)
        for chunk in (512, 0):
            with pytest.raises(pa.PaError):
                pa.pa_paged_attention_prefill(1 << 26, 1 << 27, kv, 1 << 28, 3125, 49488, chunk,
                                              32, scale, 1 << 29, big)
        for d, p in ((dec, pf), (empty_dec, empty_pf)):
            with pytest.raises(pa.PaError):
                pa.pa_paged_attention_mixed(d, p, kv, 32, scale, 1 << 29, big)
    # the smallest positive and the largest finite scale are accepted (empty
    # calls: nothing is launched)
    for scale in (1e-30, 3.4028234e38):
        pa.pa_paged_attention_decode(1 << 21, 1 << 22, kv, 1 << 23, 256, 1 << 24, 0, 32, scale,
                                     512, 4096, None, 0, None, 0)
        pa.pa_paged_attention_prefill(1 << 26, 1 << 27, kv, 1 << 28, 3125, 49488, 0, 32, scale,
                                      None, 0)
        pa.pa_paged_attention_mixed(empty_dec, empty_pf, kv, 32, scale, None, 0)


def test_mixed_checks_run_before_any_launch():
    # dummy addresses, never dereferenced: every call below fails or returns
    # on the host
    kv = pa.kv_view(None, None, 64, 8, 128)
    kv.k_pool = kv.v_pool = 1 << 20
    dec = pa.decode_batch(1 << 21, 1 << 22, 1 << 23, 256, 1 << 24, 4, 512, 4096, 1 << 25, 32)
    pf = pa.prefill_chunk(1 << 26, 1 << 27, 1 << 28, 3125, 49488, 512)
    ws_dec = pa.pa_decode_workspace_bytes(4, 32, 128, 4096, 512)
    ws_pf = pa.pa_prefill_workspace_bytes(512, 32, 128, 49488)
    assert ws_dec > 0 and ws_pf > 0
    ws = pa.pa_mixed_workspace_bytes(dec, pf, 32, 128)
    assert ws == -(-ws_dec // 256) * 256 + ws_pf
    big = 1 << 40
    with pytest.raises(pa.PaError):     # unknown flag
        pa.pa_paged_attention_mixed(dec, pf, kv, 32, 0.088, 1 << 29, big, flags=2)
    with pytest.raises(pa.PaError):     # workspace too small for the prefill part
        pa.pa_paged_attention_mixed(dec, pf, kv, 32, 0.088, 1 << 29, ws - 16)
    with pytest.raises(pa.PaError):     # 30 query heads over 8 kv heads
        pa.pa_paged_attention_mixed(dec, pf, kv, 30, 0.088, 1 << 29, big)
    bad_pf = pa.prefill_chunk(1 << 26, 1 << 27, 1 << 28, 3125, 49489, 512)   # past the table
    with pytest.raises(pa.PaError):
        pa.pa_paged_attention_mixed(dec, bad_pf, kv, 32, 0.088, 1 << 29, big)
    no_list = pa.decode_batch(1 << 21, 1 << 22, 1 << 23, 256, 1 << 24, 4, 512, 4096, None, 32)
    with pytest.raises(pa.PaError):     # decode units but no work list
        pa.pa_paged_attention_mixed(no_list, pf, kv, 32, 0.088, 1 << 29, big)
    # both parts empty: nothing to launch
    empty_dec = pa.decode_batch(1 << 21, 1 << 22, 1 << 23, 256, 1 << 24, 0, 512, 4096, None, 0)
    empty_pf = pa.prefill_chunk(1 << 26, 1 << 27, 1 << 28, 3125, 49488, 0)
    assert pa.pa_mixed_workspace_bytes(empty_dec, empty_pf, 32, 128) == 0
    pa.pa_paged_attention_mixed(empty_dec, empty_pf, kv, 32, 0.088, None, 0)


def test_pool_counts_shared_blocks():
    lib = pa.pa_pool_create(8)
    try:
        pa.pa_seq_add(lib, 0)
        pa.pa_append_slots(lib, [0], [20])                 # 2 blocks
        assert pa.pa_pool_get_stats(lib)["num_shared"] == 0
        pa.pa_seq_fork(lib, 0, 1)
        assert pa.pa_pool_get_stats(lib)["num_shared"] == 2
        pa.pa_seq_fork(lib, 0, 2)                          # ref 3: still 2 shared blocks
        assert pa.pa_pool_get_stats(lib)["num_shared"] == 2
        _, copies = pa.pa_append_slots(lib, [1], [1])      # copy-on-write of the partial block
        assert len(copies) == 1 and pa.pa_pool_get_stats(lib)["num_shared"] == 2
        pa.pa_seq_free(lib, 2)                             # the partial block is now private
        assert pa.pa_pool_get_stats(lib)["num_shared"] == 1
        pa.pa_seq_free(lib, 1)
        assert pa.pa_pool_get_stats(lib)["num_shared"] == 0
        pa.pa_pool_check(lib)
    finally:
        pa.pa_pool_destroy(lib)


@pytest.mark.parametrize("seed", range(10))
def test_prefix_cache_programs_match_oracle_exactly(seed):
    """add_cached / append / register / fork / free on a small pool and a
    small token alphabet (many shared prefixes, evictions), compared with the
    oracle model after every operation."""
    from oracle.allocator import OutOfBlocks as ModelOut
    from oracle.prefix_cache import PrefixCachingPoolModel
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(10, 30))
    order = rng.permutation(n)
    lib = pa.pa_pool_create(n, order)
    ref = PrefixCachingPoolModel(n, 16, order)
    stems = [[int(t) for t in rng.integers(0, 3, size=64)] for _ in range(3)]
    toks = {}
    nid = 0

    def compare():
        pa.pa_pool_check(lib)
        ref.check()
        assert pa.pa_free_list(lib).tolist() == ref.free
        assert pa.pa_evictable_list(lib).tolist() == ref.evictable
        st = pa.pa_pool_get_stats(lib)
        assert st["num_evictable"] == len(ref.evictable)
        assert st["num_cached"] == len(ref.cache)
        assert st["num_shared"] == sum(1 for r in ref.ref if r > 1)
        assert pa.pa_num_free_blocks(lib) == ref.num_free()
        for s in ref.tables:
            tab, ln = pa.pa_seq_table(lib, s)
            assert tab.tolist() == ref.tables[s] and ln == ref.lens[s]

    def append(s, k):
        new = [int(t) for t in rng.integers(0, 3, size=k)]
        try:
            exp = ref.append([s], [k])
        except ModelOut:
            with pytest.raises(pa.OutOfBlocksError):
                pa.pa_append_slots(lib, [s], [k])
            return False
        slots, copies = pa.pa_append_slots(lib, [s], [k])
        assert slots.tolist() == exp[0]
        assert [tuple(c) for c in copies.tolist()] == exp[1]
        toks[s] += new
        return True

    try:
        for _ in range(200):
            op = int(rng.integers(0, 6))
            live = list(ref.tables)
            if op <= 1 or not live:                       # a request arrives
                stem = stems[int(rng.integers(0, 3))]
                prompt = stem[:int(rng.integers(0, 65))] + \
                    [int(t) for t in rng.integers(0, 3, size=int(rng.integers(0, 24)))]
                hit = ref.add_cached(nid, prompt)
                assert pa.pa_seq_add_cached(lib, nid, prompt) == hit
                toks[nid] = prompt[:hit]
                rest = prompt[hit:]
                if rest:
                    try:
                        exp = ref.append([nid], [len(rest)])
                    except ModelOut:
                        with pytest.raises(pa.OutOfBlocksError):
                            pa.pa_append_slots(lib, [nid], [len(rest)])
                    else:
                        slots, copies = pa.pa_append_slots(lib, [nid], [len(rest)])
                        assert slots.tolist() == exp[0]
                        assert [tuple(c) for c in copies.tolist()] == exp[1]
                        toks[nid] += rest
                if int(rng.integers(0, 4)):
                    assert pa.pa_seq_register(lib, nid, toks[nid]) == ref.register(nid, toks[nid])
                nid += 1
            elif op == 2:
                s = int(rng.choice(live))
                append(s, int(rng.integers(1, 20)))
            elif op == 3:
                s = int(rng.choice(live))
                k = int(rng.integers(0, len(toks[s]) + 1))
                assert pa.pa_seq_register(lib, s, toks[s][:k]) == ref.register(s, toks[s][:k])
            elif op == 4:
                p = int(rng.choice(live))
                pa.pa_seq_fork(lib, p, nid)
                ref.fork(p, nid)
                toks[nid] = list(toks[p])
                nid += 1
            else:
                s = int(rng.choice(live))
                pa.pa_seq_free(lib, s)
                ref.free_seq(s)
                del toks[s]
            compare()
    finally:
        pa.pa_pool_destroy(lib)


def test_prefix_cache_register_rejects_more_tokens_than_held():
    lib = pa.pa_pool_create(4)
    try:
        pa.pa_seq_add(lib, 0)
        pa.pa_append_slots(lib, [0], [20])
        with pytest.raises(pa.PaError):
            pa.pa_seq_register(lib, 0, list(range(21)))
        with pytest.raises(pa.PaError):
            pa.pa_seq_add_cached(lib, 0, list(range(16)))     # live id
        assert pa.pa_seq_register(lib, 0, list(range(20))) == 1
        assert pa.pa_seq_add_cached(lib, 1, list(range(20))) == 16
    finally:
        pa.pa_pool_destroy(lib)


@pytest.mark.parametrize("seed", range(8))
def test_scheduler_matches_oracle_exactly(seed):
    """Random arrivals on a small pool (preemptions happen): every step's
    chunks, slots, preemptions and finished requests equal the model's."""
    from oracle.scheduler import SchedulerModel
    rng = np.random.default_rng(200 + seed)
    n = int(rng.integers(16, 80))
    order = rng.permutation(n)
    budget = int(rng.integers(4, 300))
    max_running = int(rng.integers(1, 16))
    pool = pa.pa_pool_create(n, order)
    sched = pa.pa_sched_create(pool, budget, max_running)
    model = SchedulerModel(BlockPoolModel(n, 16, order), budget, max_running)
    rid = 0
    preemptions = 0
    try:
        for step in range(100000):
            if step < 150:
                for _ in range(int(rng.integers(0, 3))):
                    prompt = int(rng.integers(1, 16 * max(1, n // 3)))
                    out = int(rng.integers(1, 40))
                    model.add_request(rid, prompt, out)
                    pa.pa_sched_add_request(sched, rid, prompt, out)
                    rid += 1
            exp = model.schedule()
            got = pa.pa_sched_schedule(sched, budget, max_running)
            assert got["items"] == [tuple(i) for i in exp.items], step
            assert got["slots"].tolist() == exp.slots
            assert [tuple(c) for c in got["copies"].tolist()] == exp.copies
            assert got["preempted"] == exp.preempted
            preemptions += len(exp.preempted)
            assert pa.pa_sched_commit(sched, max_running) == model.commit()
            pa.pa_pool_check(pool)
            assert pa.pa_free_list(pool).tolist() == model.pool.free
            st = pa.pa_sched_get_stats(sched)
            assert st["n_waiting"] == len(model.waiting) and st["n_running"] == len(model.running)
            if step >= 150 and not model.waiting and not model.running:
                break
        assert st["finished"] == rid == len(model.finished)
        for r in range(rid):
            m = model.reqs[r]
            assert pa.pa_sched_request(sched, r) == (m.computed, m.generated, m.preemptions)
    finally:
        pa.pa_sched_destroy(sched)
        pa.pa_pool_destroy(pool)


def _swap_scheduler_trace(seed):
    """Swap mode on random arrivals and a small pool: every step's chunks,
    slots, preemptions, swap-outs and swap-ins (request, tokens held, blocks)
    and finished requests equal the model's."""
    from oracle.scheduler import SchedulerModel
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(16, 80))
    order = rng.permutation(n)
    budget = int(rng.integers(4, 300))
    max_running = int(rng.integers(1, 16))
    pool = pa.pa_pool_create(n, order)
    sched = pa.pa_sched_create(pool, budget, max_running)
    pa.pa_sched_set_swap(sched, True)
    model = SchedulerModel(BlockPoolModel(n, 16, order), budget, max_running, swap=True)
    rid = 0
    swaps = 0
    try:
        for step in range(100000):
            if step < 150:
                for _ in range(int(rng.integers(0, 3))):
                    prompt = int(rng.integers(1, 16 * max(1, n // 3)))
                    out = int(rng.integers(1, 40))
                    model.add_request(rid, prompt, out)
                    pa.pa_sched_add_request(sched, rid, prompt, out)
                    rid += 1
            exp = model.schedule()
            got = pa.pa_sched_schedule(sched, budget, max_running)
            assert got["items"] == [tuple(i) for i in exp.items], step
            assert got["slots"].tolist() == exp.slots
            assert [tuple(c) for c in got["copies"].tolist()] == exp.copies
            assert got["preempted"] == exp.preempted
            ops = pa.pa_sched_swaps(sched)
            exp_ops = [(r, "out", ln, b) for r, b, ln in exp.swap_out] + \
                      [(r, "in", ln, b) for r, b, ln in exp.swap_in]
            assert [(r, k, ln, b.tolist()) for r, k, ln, b in ops] == exp_ops, step
            swaps += len(ops)
            assert pa.pa_sched_commit(sched, max_running) == model.commit()
            pa.pa_pool_check(pool)
            assert pa.pa_free_list(pool).tolist() == model.pool.free
            st = pa.pa_sched_get_stats(sched)
            assert (st["n_waiting"], st["n_running"], st["n_swapped"]) == \
                (len(model.waiting), len(model.running), len(model.swapped))
            if step >= 150 and not (model.waiting or model.running or model.swapped):
                break
        assert st["finished"] == rid == len(model.finished)
        for r in range(rid):
            m = model.reqs[r]
            assert pa.pa_sched_request(sched, r) == (m.computed, m.generated, m.preemptions)
        with pytest.raises(pa.PaError):       # the planned step's list is gone after commit
            pa.pa_sched_swaps(sched)
    finally:
        pa.pa_sched_destroy(sched)
        pa.pa_pool_destroy(pool)
    return swaps


@pytest.mark.parametrize("seed", range(8))
def test_swap_scheduler_matches_oracle_exactly(seed):
    _swap_scheduler_trace(seed)


def test_swap_scheduler_traces_do_swap():
    # the traces are tight enough that requests are swapped out and back in
    assert sum(_swap_scheduler_trace(k) for k in range(8)) > 10


def test_swap_mode_switch_checks():
    """Swap mode can change only between steps, and cannot be switched off
    while requests are swapped out (they could never resume)."""
    pool = pa.pa_pool_create(5)
    sched = pa.pa_sched_create(pool, 64, 8)
    try:
        pa.pa_sched_set_swap(sched, True)
        pa.pa_sched_add_request(sched, 0, 32, 40)
        pa.pa_sched_add_request(sched, 1, 32, 40)
        swapped = False
        for _ in range(40):
            pa.pa_sched_schedule(sched, 64, 8)
            with pytest.raises(pa.PaError):          # a plan is open
                pa.pa_sched_set_swap(sched, False)
            pa.pa_sched_commit(sched, 8)
            if pa.pa_sched_get_stats(sched)["n_swapped"]:
                swapped = True
                with pytest.raises(pa.PaError):      # request 1 is swapped out
                    pa.pa_sched_set_swap(sched, False)
                break
        assert swapped
        with pytest.raises(pa.PaError):              # no plan open
            pa.pa_sched_swaps(sched)
    finally:
        pa.pa_sched_destroy(sched)
        pa.pa_pool_destroy(pool)


def test_scheduler_argument_checks():
    pool = pa.pa_pool_create(4)
    sched = pa.pa_sched_create(pool, 16, 2)
    try:
        with pytest.raises(pa.PaError):
            pa.pa_sched_add_request(sched, 0, 60, 6)          # 65 tokens > 4 blocks
        pa.pa_sched_add_request(sched, 0, 60, 5)
        with pytest.raises(pa.PaError):
            pa.pa_sched_add_request(sched, 0, 1, 1)           # duplicate id
        with pytest.raises(pa.PaError):
            pa.pa_sched_schedule(sched, 8, 2)                 # slot buffer below the budget
        pa.pa_sched_schedule(sched, 16, 2)
        with pytest.raises(pa.PaError):
            pa.pa_sched_schedule(sched, 16, 2)                # previous plan not committed
        pa.pa_sched_commit(sched, 2)
    finally:
        pa.pa_sched_destroy(sched)
        pa.pa_pool_destroy(pool)
