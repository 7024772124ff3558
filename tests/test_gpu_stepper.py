"""The decode step the benchmark times, as its stepper runs it: slots
reserved on the host, lengths and work list moved from pinned host memory
and the device block table brought up to date (its changed entries only)
by one pa_stage_update launch, the step's K/V stored, then the work-list
decode (ta-paperlens "LLM serving from scratch", scheduler skeleton: blocks
are reserved for every running request before the forward pass;
"fragmentation and PagedAttention": the kernel reads K/V through the block
table).

The first step must equal the fp64 oracle's decode of the same workload
step; later steps (the pool grown by one token per request each time) must
equal, bitwise, a decode planned from scratch on the same pool, and the
device table the host library's table of that moment.
"""
import numpy as np
import pytest
import torch

from gpu_util import assert_close, log, oracle_run, shared_reference, shared_workload
from oracle import decode_reference

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", ["2", "3"])
def test_decode_stepper_matches_oracle_then_fresh_plans(cfg):
    """Config 2 runs 20 steps (every request takes a new block at least once,
    and one step is forced to copy the whole table again); config 3 runs 3."""
    from pagedattention_block_paged_reshape_amd.cache import (DecodePlan, PagedKVCache,
                                                              run_program)
    from pagedattention_block_paged_reshape_amd.stepper import DecodeStepper
    w = shared_workload(cfg)
    assert list(w.step_ids) == list(w.decode_ids) and set(np.asarray(w.step_n_new)) == {1}
    dev = torch.device("cuda:0")
    steps = 20 if cfg == "2" else 3
    extra = w.batch * (steps // 16 + 2)
    free_order = np.concatenate([np.arange(w.num_blocks, w.num_blocks + extra, dtype=np.int32),
                                 np.asarray(w.free_order, dtype=np.int32)])
    cache = PagedKVCache(w.num_blocks + extra, w.n_kv, w.d, free_order, dev)
    dk = torch.from_numpy(w.setup_k).to(dev)
    dv = torch.from_numpy(w.setup_v).to(dev)
    run_program(cache, w.setup, dk, dv)
    del dk, dv
    sk = torch.from_numpy(w.step_k[:w.batch]).to(dev)
    sv = torch.from_numpy(w.step_v[:w.batch]).to(dev)
    q = torch.from_numpy(w.q).to(dev)
    cap = max(cache.seq_len(int(s)) for s in w.decode_ids) + steps
    stepper = DecodeStepper(cache, w.decode_ids, w.n_q, w.scale, cap, 512)
    log(f"[stepper] config {cfg}: B={w.batch}, cap {cap}")

    out = stepper.step(q, sk, sv).clone()
    torch.cuda.synchronize()
    if cfg == "3":
        ref = shared_reference(3, "decode")
    else:
        ref = decode_reference(w, oracle_run(w))
    err = assert_close(out, ref, f"config {cfg} stepper decode")
    log(f"[stepper] config {cfg} step 1: max err {err:.2e}")

    import pagedattention_block_paged_reshape_amd._lib as L
    forced = 10 if steps >= 10 else None
    for i in range(2, steps + 1):
        if i == forced:
            stepper.upd_cap = 0                 # more changes than the list holds: whole table
        out = stepper.step(q, sk, sv).clone()
        torch.cuda.synchronize()
        if i == forced:
            stepper.upd_cap = max(1024, 4 * w.batch)
        lens = stepper.last_lens
        assert (lens == np.asarray([cache.seq_len(int(s)) for s in w.decode_ids])).all()
        tab, _ = L.pa_block_tables(cache.pool, np.asarray(w.decode_ids, dtype=np.int64),
                                   stepper.max_blocks)
        assert np.array_equal(stepper.d_tab.cpu().numpy(), tab), f"step {i}: device table"
        plan = DecodePlan(cache, w.decode_ids, w.n_q, w.scale, 512)
        fresh = plan.run(q).clone()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), fresh.view(torch.int16)), f"step {i}"
        log(f"[stepper] config {cfg} step {i}: bitwise equal to a fresh plan")
    assert stepper.full_uploads == (2 if forced else 1)
    if cfg == "2":
        assert stepper.updated_entries >= w.batch   # every request took a new block
    log(f"[stepper] config {cfg}: {stepper.full_uploads} whole-table copies, "
        f"{stepper.updated_entries} entries updated in {steps} steps")


def test_fp8_decode_stepper_matches_oracle_then_fresh_plans():
    """The same stepper over FP8 (E4M3) pools on config 2: the step's K/V are
    quantised by the store, the first step matches the oracle attending the
    dequantised pool, and 17 more steps (every request takes a new block)
    equal fresh plans bitwise, with the device table equal to the host
    library's each time."""
    import pagedattention_block_paged_reshape_amd._lib as L
    from pagedattention_block_paged_reshape_amd.cache import (DecodePlan, PagedKVCache,
                                                              run_program)
    from pagedattention_block_paged_reshape_amd.stepper import DecodeStepper
    k_scale, v_scale = 5.5 / 448, 4.75 / 448
    w = shared_workload("2")
    dev = torch.device("cuda:0")
    steps = 18
    extra = w.batch * (steps // 16 + 2)
    free_order = np.concatenate([np.arange(w.num_blocks, w.num_blocks + extra, dtype=np.int32),
                                 np.asarray(w.free_order, dtype=np.int32)])
    cache = PagedKVCache(w.num_blocks + extra, w.n_kv, w.d, free_order, dev, kv_dtype="fp8",
                         k_scale=k_scale, v_scale=v_scale)
    dk = torch.from_numpy(w.setup_k).to(dev)
    dv = torch.from_numpy(w.setup_v).to(dev)
    run_program(cache, w.setup, dk, dv)
    del dk, dv
    sk = torch.from_numpy(w.step_k[:w.batch]).to(dev)
    sv = torch.from_numpy(w.step_v[:w.batch]).to(dev)
    q = torch.from_numpy(w.q).to(dev)
    cap = max(cache.seq_len(int(s)) for s in w.decode_ids) + steps
    stepper = DecodeStepper(cache, w.decode_ids, w.n_q, w.scale, cap, 512)
    out = stepper.step(q, sk, sv).clone()
    torch.cuda.synchronize()
    ref = decode_reference(w, oracle_run(w, "fp8", k_scale, v_scale))
    err = assert_close(out, ref, "fp8 config 2 stepper decode")
    ids = np.asarray(w.decode_ids, dtype=np.int64)
    for i in range(2, steps + 1):
        out = stepper.step(q, sk, sv).clone()
        torch.cuda.synchronize()
        tab, _ = L.pa_block_tables(cache.pool, ids, stepper.max_blocks)
        assert np.array_equal(stepper.d_tab.cpu().numpy(), tab), f"step {i}: device table"
        fresh = DecodePlan(cache, w.decode_ids, w.n_q, w.scale, 512).run(q).clone()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), fresh.view(torch.int16)), f"step {i}"
    assert stepper.full_uploads == 1 and stepper.updated_entries >= w.batch
    log(f"[stepper] fp8 config 2: step 1 max err {err:.2e}; {steps - 1} more steps bitwise "
        f"equal to fresh plans, {stepper.updated_entries} table entries updated")


def test_stage_update_copies_and_applies_updates_exactly():
    """pa_stage_update: the dense bytes as pa_stage_copy moves them, and
    every in-range (index, value) pair applied to the target, from pinned
    host memory; out-of-range indices are skipped and nothing else changes."""
    import pagedattention_block_paged_reshape_amd as pa
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    rng = np.random.default_rng(11)
    n_dense, n_target = 4096 + 64, 70000
    host = torch.empty(n_dense + 2 * 100000, dtype=torch.int32, pin_memory=True)
    h = host.numpy()
    h[:] = rng.integers(-2**31, 2**31 - 1, h.size, dtype=np.int64).astype(np.int32)
    base = pa.pa_host_device_pointer(host)
    for n_bytes, n_upd in ((4 * n_dense, 5000), (0, 777), (4 * n_dense, 0), (64, 60000),
                           (4 * n_dense, 1)):
        idx = rng.permutation(n_target + 500)[:n_upd].astype(np.int32) - 250  # some out of range
        vals = rng.integers(-2**31, 2**31 - 1, n_upd, dtype=np.int64).astype(np.int32)
        pairs = h[n_dense:n_dense + 2 * n_upd].reshape(n_upd, 2)
        pairs[:, 0] = idx
        pairs[:, 1] = vals
        dst = torch.full((n_dense,), -7, dtype=torch.int32, device=dev)
        target0 = rng.integers(-2**31, 2**31 - 1, n_target, dtype=np.int64).astype(np.int32)
        target = torch.from_numpy(target0.copy()).to(dev)
        pa.pa_stage_update(base, dst, n_bytes, base + 4 * n_dense, n_upd, target, n_target,
                           stream)
        torch.cuda.synchronize()
        got = dst.cpu().numpy()
        k = n_bytes // 4
        assert np.array_equal(got[:k], h[:k]) and (got[k:] == -7).all()
        want = target0.copy()
        ok = (idx >= 0) & (idx < n_target)
        want[idx[ok]] = vals[ok]
        assert np.array_equal(target.cpu().numpy(), want)
        log(f"stage update: {n_bytes} bytes, {n_upd} updates ({int(ok.sum())} in range)")


def test_stage_copy_moves_pinned_host_bytes_exactly():
    """pa_stage_copy: whole 16-byte chunks from pinned host memory (through
    pa_host_device_pointer) into device memory, bit for bit, and nothing past
    the requested size."""
    import pagedattention_block_paged_reshape_amd as pa
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(7)
    n_int = (1 << 20) + 64
    host = torch.empty(n_int, dtype=torch.int32, pin_memory=True)
    host.numpy()[:] = rng.integers(-2**31, 2**31 - 1, n_int, dtype=np.int64).astype(np.int32)
    src = pa.pa_host_device_pointer(host)
    assert src != 0
    stream = torch.cuda.current_stream(dev)
    for nbytes in (16, 48, 4096, 65536 + 16, 4 * n_int):
        dst = torch.full((n_int,), -7, dtype=torch.int32, device=dev)
        pa.pa_stage_copy(src, dst, nbytes, stream)
        torch.cuda.synchronize()
        got = dst.cpu().numpy()
        k = nbytes // 4
        log(f"stage copy {nbytes} bytes")
        assert np.array_equal(got[:k], host.numpy()[:k])
        assert (got[k:] == -7).all()
    # an interior pointer of the pinned allocation maps to the same offset
    assert pa.pa_host_device_pointer(host.data_ptr() + 4096) == src + 4096


def test_host_device_pointer_rejects_pageable_memory_and_the_runtime_stays_usable():
    """Memory the runtime does not hold as pinned gets PA_ERR_INVALID (its
    sticky runtime error cleared), and later launches still run."""
    import pagedattention_block_paged_reshape_amd as pa
    import pagedattention_block_paged_reshape_amd._lib as L
    pageable = np.zeros(4096, dtype=np.int32)
    with pytest.raises(pa.PaError) as e:
        pa.pa_host_device_pointer(pageable.ctypes.data)
    assert e.value.status == L.PA_ERR_INVALID
    host = torch.arange(1024, dtype=torch.int32).pin_memory()
    dst = torch.zeros(1024, dtype=torch.int32, device="cuda:0")
    pa.pa_stage_copy(pa.pa_host_device_pointer(host), dst, 4096, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), host)


def test_serving_staging_ring_grows_and_moves_every_section():
    """The serving loop's staging: sections of both int widths, a buffer
    that has to grow mid-step, and three steps around the ring; every
    device view equals its host array."""
    from pagedattention_block_paged_reshape_amd.serve import _Staging
    dev = torch.device("cuda:0")
    st = _Staging(dev, nbytes=256, depth=2)
    rng = np.random.default_rng(11)
    stream = torch.cuda.current_stream(dev)
    for step in range(3):
        arrays = [rng.integers(-2**31, 2**31 - 1, n).astype(dt)
                  for n, dt in ((5, np.int64), (3, np.int32), (4000, np.int32), (1, np.int64),
                                (0, np.int32), (777 + step, np.int64))]
        st.begin()
        idx = [st.add(a) for a in arrays]
        views = st.upload(stream)
        torch.cuda.synchronize()
        for i, a in zip(idx, arrays):
            assert np.array_equal(views[i].cpu().numpy(), a), (step, i)
