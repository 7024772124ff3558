#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 3] [--kv-dtype fp8]

A step is one pass of the whole decode hot path for the batch: reserve one
slot per request on the host block manager, store the step's new K/V into the
paged pool, refresh the device block tables, and run paged decode attention
(split-K work-list kernel + reduce).  The default workload is the
Llama-3-70B-shaped decode layer: 256 requests, 64 query / 8 KV heads,
head_dim 128, 16-token blocks, lengths lognormal(median 1000) clipped to
[16, 4096], split-K partitions of 512 tokens, block tables scattered over the
pool.  Inputs are seeded synthetic fp16 N(0,1) data, resident in HBM before
timing starts.

Prints one JSON line.  ``value`` is decode tokens/s per layer (requests
advanced per second).  ``roofline`` reports the decode launch (work-list +
reduce kernels, timed with HIP events on the stream they run on) against the
8 TB/s HBM peak using algorithmic bytes: every K and V byte of every attended
token once per KV head, plus Q, O, block tables and lengths.  With
``--kv-dtype fp8`` the pools hold E4M3 codes (one byte per value, one scale
per pool) and the same step runs the FP8 store and decode entry points.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["pagedattention_block_paged_reshape_amd/csrc/decode_core.h",
                  "pagedattention_block_paged_reshape_amd/csrc/decode.hip",
                  "pagedattention_block_paged_reshape_amd/csrc/pa_device.h"]
PREFILL_SOURCES = ["pagedattention_block_paged_reshape_amd/csrc/prefill_tile.h",
                   "pagedattention_block_paged_reshape_amd/csrc/prefill.hip",
                   "pagedattention_block_paged_reshape_amd/csrc/pa_device.h"]
TRAFFIC_FILES = {"fp16": os.path.join(PROFILES, "decode_llama3-70b_traffic.md"),
                 "fp8": os.path.join(PROFILES, "decode_llama3-70b_fp8_traffic.md")}
PREFILL_TRAFFIC_FILES = {"fp16": os.path.join(PROFILES, "prefill_long-context-chunk_traffic.md")}
# FP8 pools: one scale per pool, about max |x| / 448 for the N(0, 1) rows
FP8_K_SCALE, FP8_V_SCALE = 5.5 / 448, 4.75 / 448


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash(sources=KERNEL_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(kv_dtype: str = "fp16", prefill: bool = False):
    """HBM bytes per decode (or prefill) launch from the committed rocprofv3
    counter summary, if it was taken on the current kernel sources."""
    path = (PREFILL_TRAFFIC_FILES if prefill else TRAFFIC_FILES).get(kv_dtype)
    if path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    sources = PREFILL_SOURCES if prefill else KERNEL_SOURCES
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash(sources):
        return None
    return float(m_bytes.group(1))


def algorithmic_decode_bytes(lens, n_q, n_kv, d, kv_bytes: int = 2) -> int:
    lens = np.asarray(lens, dtype=np.int64)
    kv = int(lens.sum()) * 2 * n_kv * d * kv_bytes       # K and V once per KV head
    qo = 2 * len(lens) * n_q * d * 2                     # Q in, O out (fp16)
    tables = 4 * int(((lens + 15) // 16).sum())          # block ids read
    return kv + qo + tables + 4 * len(lens)              # + lengths


def cpu_baseline(w, budget_s: float, steps_done: int, kv_dtype: str = "fp16"):
    """The fp64 oracle (as written, untuned) doing the same decode step:
    append one token per request, store its K/V, attend over every request."""
    from oracle import decode_reference, run_setup
    log("[bench] cpu_baseline: building the oracle's pool model (not timed)")
    st = run_setup(w, kv_dtype=kv_dtype, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    ids, ones = w.step_ids.tolist(), [1] * w.batch
    for _ in range(steps_done):                  # reach the GPU's final lengths
        st.alloc.append(ids, ones)
    t0, c0 = time.perf_counter(), time.process_time()
    reps = 0
    while True:
        slots, copies = st.alloc.append(ids, ones)
        st.pool.copy(copies)
        st.pool.write(w.step_k, w.step_v, slots)
        decode_reference(w, st)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    cpu = time.process_time() - c0
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas = None
    return {
        "value": reps * w.batch / el,
        "unit": "decode tokens/s per layer",
        "cores": max(1, int(round(cpu / el))),
        "kind": "oracle",
        "sample": f"{reps} full decode steps of the same workload ({w.batch} requests each: "
                  f"append + store{' (E4M3 encode)' if kv_dtype == 'fp8' else ''} + fp64 "
                  f"attention) in {el:.1f} s wall; BLAS pool "
                  f"{blas} threads, cpu/wall = {cpu / el:.2f}",
    }


def prefill_flops(q_start: int, chunk_len: int, n_q: int, d: int) -> int:
    """Matrix-core flops of one causal chunk: row r sees q_start + r + 1 keys;
    per (row, head, key) 2*d for q.k and 2*d for p.v."""
    pairs = chunk_len * q_start + chunk_len * (chunk_len + 1) // 2
    return 4 * d * n_q * pairs


def cpu_prefill_baseline(w, budget_s: float):
    """The fp64 oracle's causal chunk attention on a bounded sample of the
    same chunk: all 512 rows for as many query heads as the budget allows."""
    from oracle import prefill_reference, run_setup, run_step
    log("[bench] cpu_baseline: building the oracle's pool model (not timed)")
    st = run_setup(w)
    run_step(w, st)
    pf = w.prefill
    t0, c0 = time.perf_counter(), time.process_time()
    heads = 0
    while True:
        prefill_reference(w, st, heads=[heads % w.n_q])
        heads += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    cpu = time.process_time() - c0
    flops = prefill_flops(pf.q_start, pf.chunk_len, 1, w.d) * heads
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": max(1, int(round(cpu / el))),
        "kind": "oracle",
        "sample": f"{heads} single-head passes (cycling over the chunk's {w.n_q} query heads; all {pf.chunk_len} rows, "
                  f"{pf.q_start + pf.chunk_len} keys each) in {el:.1f} s wall, "
                  f"cpu/wall = {cpu / el:.2f}",
    }


def clock_warmup(fn, ms: float) -> int:
    """Launch fn back to back for about `ms` milliseconds, untimed: the GPU
    only reaches its sustained clocks after tens of milliseconds of load
    (measured: a prefill launch takes ~20 % longer in the first ~50 ms).
    Returns the number of launches."""
    import torch
    n = 0
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        n += 10
    return n


def bench_serve(args):
    """Continuous batching over many steps with arrivals: the C++ scheduler
    plans each step (decode first, chunked prefill, preemption when the pool
    runs out) and the step runs reshape_and_cache, one decode launch and the
    prefill chunks.  Llama-3-70B-shaped layer (64/8 heads, head_dim 128);
    256 requests, prompts lognormal(median 1000) clipped to [16, 4096],
    outputs uniform in [64, 256], arriving over the first 64 steps; the pool
    holds half of what all requests would need at once."""
    import torch
    from synth.serving import make_trace, token_rows_kvq
    from pagedattention_block_paged_reshape_amd.cache import PagedKVCache
    from pagedattention_block_paged_reshape_amd.serve import ServingLoop
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n_q, n_kv, d = 64, 8, 128
    tr = make_trace(256, seed=2003, arrive_over=64)
    need = sum(-(-(p + o) // 16) for p, o in zip(tr.prompt, tr.output))
    blocks = need // 2
    order = np.random.default_rng(2003).permutation(blocks).astype(np.int32)
    cache = PagedKVCache(blocks, n_kv, d, order, dev)
    rows_fn = lambda r, p, wkv, wq: token_rows_kvq(r, p, wkv, wq, xp=torch)
    budget, max_running = 8192, 256

    def run(loop, trace):
        nxt, step = 0, 0
        while True:
            while nxt < len(trace.prompt) and trace.arrival[nxt] <= step:
                loop.add(nxt, trace.prompt[nxt], trace.output[nxt])
                nxt += 1
            loop.step()
            step += 1
            st = loop.sched_stats()
            if (nxt == len(trace.prompt) and st["n_waiting"] == 0 and st["n_running"] == 0
                    and st["n_swapped"] == 0):
                return step

    # clock warm-up on a small trace of the same shape (not timed)
    warm = ServingLoop(cache, n_q, 1.0 / np.sqrt(d), budget, max_running, rows_fn=rows_fn,
                       mixed=args.mixed)
    run(warm, make_trace(32, seed=1, arrive_over=4))
    warm.close()
    torch.cuda.synchronize()
    loop = ServingLoop(cache, n_q, 1.0 / np.sqrt(d), budget, max_running, rows_fn=rows_fn,
                       swap=args.swap, mixed=args.mixed)
    t0 = time.perf_counter()
    steps = run(loop, tr)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    out_tokens = sum(tr.output)
    st = loop.stats
    log(f"[bench] serve: {steps} steps in {wall * 1e3:.1f} ms; {st}")
    result = {
        "metric": "serving: generated tokens/s per layer (continuous batching with chunked "
                  "prefill and preemption)",
        "value": round(out_tokens / wall, 1),
        "unit": "generated tokens/s per layer",
        "n_gpus": 1,
        "steps": steps,
        "warmup": 0,
        "ms_per_step": round(wall * 1e3 / steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": "256 requests, Llama-3-70B-shaped layer (64/8 heads, head_dim 128), "
                        "prompts lognormal(median 1000) in [16, 4096], outputs U[64, 256], "
                        "arrivals over 64 steps, pool = half of the peak demand",
            "pool_blocks": blocks, "token_budget": budget, "max_running": max_running,
            "prefill_tokens": st["prefill_tokens"], "decode_tokens": st["decode_tokens"],
            "preemptions": st["preempted"], "generated_tokens": out_tokens,
            "preemption_mode": "swap" if args.swap else "recompute",
            "mixed_launches": bool(args.mixed),
            "swapped_out": st["swapped_out"], "swapped_in": st["swapped_in"],
        },
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)
    loop.close()


def measure_prefill(args, kv_dtype: str):
    """Time the causal prefill chunk of workload 5 (512 rows at offset 49,488
    of a 50,000-token prompt, 32/8 heads, head_dim 128) after the clock
    warm-up: ``args.prefill_steps`` launches, each bracketed by HIP events on
    the stream it runs on.  Returns the launch times (ms), the wall time of
    the timed launches, the algorithmic flops and the workload."""
    import torch
    from synth import make_workload
    from pagedattention_block_paged_reshape_amd.cache import (PagedKVCache, PrefillPlan,
                                                              run_program)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] generating workload 5")
    w = make_workload("5")
    pf = w.prefill
    cache = PagedKVCache(w.num_blocks, w.n_kv, w.d, w.free_order, dev, kv_dtype=kv_dtype,
                         k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    dk = torch.from_numpy(w.setup_k).to(dev)
    dv = torch.from_numpy(w.setup_v).to(dev)
    run_program(cache, w.setup, dk, dv)
    del dk, dv
    cache.append(w.step_ids, w.step_n_new, torch.from_numpy(w.step_k).to(dev),
                 torch.from_numpy(w.step_v).to(dev))
    plan = PrefillPlan(cache, pf.seq_id, pf.q_start, pf.chunk_len, w.n_q, w.scale)
    q = torch.from_numpy(pf.q).to(dev)
    stream = torch.cuda.current_stream(dev)
    n_warm = clock_warmup(lambda: plan.run(q, stream), args.warm_ms)
    log(f"[bench] prefill clock warm-up: {n_warm} launches in ~{args.warm_ms:.0f} ms")
    for _ in range(args.warmup):
        plan.run(q, stream)
    torch.cuda.synchronize()
    n = args.prefill_steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    t0 = time.perf_counter()
    for e in ev:
        e[0].record(stream)
        plan.run(q, stream)
        e[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    flops = prefill_flops(pf.q_start, pf.chunk_len, w.n_q, w.d)
    log(f"[bench] prefill launch mean {ms.mean() * 1e3:.1f} us (p50 {np.median(ms) * 1e3:.1f}); "
        f"{flops / 1e9:.1f} GFLOP -> {flops / (ms.mean() * 1e-3) / 1e12:.1f} TFLOP/s")
    del cache, plan, q
    torch.cuda.empty_cache()
    return ms, wall, flops, w


def prefill_roofline(ms, flops, kv_dtype: str) -> dict:
    achieved = flops / (ms.mean() * 1e-3) / 1e12
    fp8 = kv_dtype == "fp8"
    return {
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": MFMA_F16_PEAK_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
        "traffic": recorded_traffic(kv_dtype, prefill=True),
        "kernel": f"pa_paged_attention_prefill{'_fp8' if fp8 else ''} "
                  f"({'prefill_chunk_kernel' if fp8 else 'prefill_chunk_pp_kernel'} + "
                  "prefill_reduce_kernel)",
        "algorithmic_flops_per_launch": flops,
        "launch_us_mean": round(float(ms.mean()) * 1e3, 2),
        "launch_us_p50": round(float(np.median(ms)) * 1e3, 2),
        "launch_us_p99": round(float(np.percentile(ms, 99)) * 1e3, 2),
        "kernel_source_sha256": kernel_source_hash(PREFILL_SOURCES),
    }


def prefill_workload_text(w) -> str:
    pf = w.prefill
    return (f"config 5 chunk ({w.name}): causal chunk of {pf.chunk_len} query rows at offset "
            f"{pf.q_start} of a {pf.q_start + pf.chunk_len}-token prompt, {w.n_q}/{w.n_kv} "
            f"heads, head_dim {w.d}, block 16, pool {w.num_blocks} blocks scattered")


def bench_prefill(args):
    """Causal chunked prefill over the paged cache: the 512-token chunk at
    offset 49,488 of a 50,000-token prompt (32/8 heads, head_dim 128)."""
    import torch
    ms, wall, flops, w = measure_prefill(args, args.kv_dtype)
    pf = w.prefill
    n = len(ms)
    result = {
        "metric": "paged prefill chunk attention TFLOP/s (% of fp16 MFMA peak)",
        "value": round(flops * n / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / n, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": prefill_workload_text(w),
            "chunk": pf.chunk_len,
            "q_start": pf.q_start,
            "kv_dtype": args.kv_dtype,
            "clock_warmup_ms": args.warm_ms,
        },
        "roofline": prefill_roofline(ms, flops, args.kv_dtype),
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_prefill_baseline(w, args.cpu_budget)
    print(json.dumps(result), flush=True)


def bench_mixed(args):
    """The long-context mixed step of workload 5: 8 decode requests at 32,768
    tokens and the 512-row causal prefill chunk at offset 49,488 of a
    50,000-token prompt, over one pool.  Times the one-launch mixed entry point
    against the same work as separate decode and prefill launches on one
    stream (and each part alone).  With ``--kv-dtype fp8`` the pool holds
    E4M3 codes and the _fp8 entry points run."""
    import torch
    from synth import make_workload
    from pagedattention_block_paged_reshape_amd.cache import (DecodePlan, MixedPlan, PagedKVCache,
                                                              PrefillPlan, run_program)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("[bench] generating workload 5")
    w = make_workload("5")
    pf = w.prefill
    fp8 = args.kv_dtype == "fp8"
    cache = PagedKVCache(w.num_blocks, w.n_kv, w.d, w.free_order, dev, kv_dtype=args.kv_dtype,
                         k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    dk = torch.from_numpy(w.setup_k).to(dev)
    dv = torch.from_numpy(w.setup_v).to(dev)
    run_program(cache, w.setup, dk, dv)
    del dk, dv
    cache.append(w.step_ids, w.step_n_new, torch.from_numpy(w.step_k).to(dev),
                 torch.from_numpy(w.step_v).to(dev))
    dplan = DecodePlan(cache, w.decode_ids, w.n_q, w.scale, args.partition)
    pplan = PrefillPlan(cache, pf.seq_id, pf.q_start, pf.chunk_len, w.n_q, w.scale)
    mplan = MixedPlan(cache, w.decode_ids, pf.seq_id, pf.q_start, pf.chunk_len, w.n_q, w.scale,
                      args.partition)
    qd = torch.from_numpy(w.q).to(dev)
    qp = torch.from_numpy(pf.q).to(dev)
    stream = torch.cuda.current_stream(dev)

    def separate():
        pplan.run(qp, stream)
        dplan.run(qd, stream)

    def mixed():
        mplan.run(qd, qp, stream)

    def time_it(fn, n):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        t0 = time.perf_counter()
        for e in ev:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return np.array([a.elapsed_time(b) * 1e3 for a, b in ev]), wall

    n_warm = clock_warmup(mixed, args.warm_ms)
    log(f"[bench] clock warm-up: {n_warm} mixed launches in ~{args.warm_ms:.0f} ms")
    t_dec, _ = time_it(lambda: dplan.run(qd, stream), args.steps)
    t_pf, _ = time_it(lambda: pplan.run(qp, stream), args.steps)
    t_sep, _ = time_it(separate, args.steps)
    t_mix, wall = time_it(mixed, args.steps)
    flops = prefill_flops(pf.q_start, pf.chunk_len, w.n_q, w.d)
    dec_bytes = algorithmic_decode_bytes(dplan.lens.cpu().numpy(), w.n_q, w.n_kv, w.d,
                                         kv_bytes=1 if fp8 else 2)
    achieved = flops / (t_mix.mean() * 1e-6) / 1e12
    log(f"[bench] decode alone {t_dec.mean():.1f} us, prefill alone {t_pf.mean():.1f} us, "
        f"separate launches {t_sep.mean():.1f} us, mixed launch {t_mix.mean():.1f} us "
        f"(p50 {np.median(t_mix):.1f}, p99 {np.percentile(t_mix, 99):.1f})")
    result = {
        "metric": "mixed decode + prefill attention step time (config 5"
                  + (", FP8 E4M3 pool)" if fp8 else ")"),
        "value": round(float(t_mix.mean()), 2),
        "unit": "us per step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"config 5 ({w.name}): {w.batch} decode requests at "
                        f"{int(dplan.lens.max())} tokens (split-K {args.partition}) + causal "
                        f"chunk of {pf.chunk_len} rows at offset {pf.q_start} of a "
                        f"{pf.q_start + pf.chunk_len}-token prompt, {w.n_q}/{w.n_kv} heads, "
                        f"head_dim {w.d}, block 16, pool {w.num_blocks} blocks scattered",
            "kv_dtype": args.kv_dtype,
            "clock_warmup_ms": args.warm_ms,
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_F16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
            "traffic": None,
            "kernel": f"pa_paged_attention_mixed{'_fp8' if fp8 else ''} (mixed_step_kernel + mixed_prefill_reduce_kernel + decode_reduce_kernel); "
                      "achieved = the chunk's matrix-core flops over the whole mixed launch",
            "algorithmic_flops_per_launch": flops,
            "decode_algorithmic_bytes_per_launch": int(dec_bytes),
            "launch_us_mean": round(float(t_mix.mean()), 2),
            "launch_us_p50": round(float(np.median(t_mix)), 2),
            "launch_us_p99": round(float(np.percentile(t_mix, 99)), 2),
            "separate_launches_us_mean": round(float(t_sep.mean()), 2),
            "decode_alone_us_mean": round(float(t_dec.mean()), 2),
            "prefill_alone_us_mean": round(float(t_pf.mean()), 2),
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        del cache, dplan, pplan, mplan
        torch.cuda.empty_cache()
        result["cpu_baseline"] = cpu_prefill_baseline(w, args.cpu_budget)
    print(json.dumps(result), flush=True)


def copy_calibration(nbytes: int, reps: int):
    """A plain device copy of known size (for scaling HBM byte counters)."""
    import torch
    src = torch.empty(nbytes // 2, dtype=torch.float16, device="cuda:0").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-ms", type=float, default=250.0,
                    help="before the warm-up steps, launch the attention kernels on the "
                         "starting state for this long (state unchanged) so that the GPU "
                         "runs at its sustained clocks")
    ap.add_argument("--config", default="3", help="decode workload (2, 3, 4 or 5)")
    ap.add_argument("--partition", type=int, default=512)
    ap.add_argument("--kv-dtype", choices=["fp16", "fp8"], default="fp16",
                    help="KV pool type of the decode step: fp16, or FP8 E4M3 codes with one "
                         "scale per pool")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mb", type=int, default=0,
                    help="read this many MiB between steps to evict L2/MALL (a read leaves "
                         "no dirty lines behind to be written back during the next step)")
    ap.add_argument("--copy-calibration-mb", type=int, default=0)
    ap.add_argument("--prefill", action="store_true",
                    help="time the causal prefill chunk of workload 5 instead of decode")
    ap.add_argument("--prefill-steps", type=int, default=20,
                    help="timed launches of the prefill chunk (its own line, or the prefill "
                         "sub-object of the decode line)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="leave the prefill sub-object out of the decode line")
    ap.add_argument("--mixed", action="store_true",
                    help="time workload 5's decode batch and prefill chunk as one mixed "
                         "launch (and as separate launches) instead of the decode step; "
                         "with --serve: run each step's decode batch and first prefill chunk "
                         "as one mixed launch")
    ap.add_argument("--swap", action="store_true",
                    help="with --serve: preempt by swapping to host memory instead of "
                         "recomputing")
    ap.add_argument("--serve", action="store_true",
                    help="continuous-batching serving run (scheduler + kernels) instead of "
                         "the decode step")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the kernels shard by request or KV head with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration_mb:
        copy_calibration(args.copy_calibration_mb << 20, 5)
        return
    if args.prefill:
        bench_prefill(args)
        return
    if args.serve:
        bench_serve(args)
        return
    if args.mixed:
        bench_mixed(args)
        return

    from synth import make_workload
    from pagedattention_block_paged_reshape_amd.cache import PagedKVCache, run_program
    from pagedattention_block_paged_reshape_amd.stepper import DecodeStepper

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] generating workload {args.config}")
    w = make_workload(args.config)
    total_steps = args.warmup + args.steps
    # room for the timed steps' appends (one token per request per step, plus
    # a copy-on-write per request): extra blocks go to the bottom of the free
    # stack, so the workload's own allocations are unchanged
    extra = w.batch * (total_steps // 16 + 2)
    free_order = np.concatenate([np.arange(w.num_blocks, w.num_blocks + extra, dtype=np.int32),
                                 np.asarray(w.free_order, dtype=np.int32)])
    fp8 = args.kv_dtype == "fp8"
    cache = PagedKVCache(w.num_blocks + extra, w.n_kv, w.d, free_order, dev,
                         kv_dtype=args.kv_dtype, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE)
    log("[bench] uploading and storing the cached K/V through reshape_and_cache")
    dk = torch.from_numpy(w.setup_k).to(dev)
    dv = torch.from_numpy(w.setup_v).to(dev)
    run_program(cache, w.setup, dk, dv)
    del dk, dv
    step_k = torch.from_numpy(w.step_k[:w.batch]).to(dev)
    step_v = torch.from_numpy(w.step_v[:w.batch]).to(dev)
    q = torch.from_numpy(w.q).to(dev)
    lens0 = np.array([cache.seq_len(int(s)) for s in w.decode_ids])
    cap = int(lens0.max()) + total_steps
    stepper = DecodeStepper(cache, w.decode_ids, w.n_q, w.scale, cap, args.partition)
    stream = torch.cuda.current_stream(dev)
    flush = None
    if args.flush_mb:
        flush = torch.ones((args.flush_mb << 20) // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    if args.warm_ms > 0:
        from pagedattention_block_paged_reshape_amd.cache import DecodePlan
        warm_plan = DecodePlan(cache, w.decode_ids, w.n_q, w.scale, args.partition,
                               worklist=True)
        n_warm = clock_warmup(lambda: warm_plan.run(q, stream), args.warm_ms)
        log(f"[bench] clock warm-up: {n_warm} attention launches in ~{args.warm_ms:.0f} ms")
        del warm_plan
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        stepper.step(q, step_k, step_v, stream)
    torch.cuda.synchronize()

    ev = [{"cache": (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)),
           "decode": (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))}
          for _ in range(args.steps)]
    bytes_per_step = []
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if flush is not None:
            flush_sink = flush.sum()
        stepper.step(q, step_k, step_v, stream, events=ev[i])
        bytes_per_step.append(algorithmic_decode_bytes(stepper.last_lens, w.n_q, w.n_kv, w.d,
                                                       1 if fp8 else 2))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    dec_ms = np.array([e["decode"][0].elapsed_time(e["decode"][1]) for e in ev])
    cache_ms = np.array([e["cache"][0].elapsed_time(e["cache"][1]) for e in ev])
    dec_bytes = float(np.mean(bytes_per_step))
    achieved = dec_bytes / (dec_ms.mean() * 1e-3) / 1e9
    tokens_per_s = w.batch * args.steps / wall
    log(f"[bench] wall {wall * 1e3:.2f} ms for {args.steps} steps; decode launch mean "
        f"{dec_ms.mean() * 1e3:.1f} us (p50 {np.median(dec_ms) * 1e3:.1f}, p99 "
        f"{np.percentile(dec_ms, 99) * 1e3:.1f}); reshape_and_cache {cache_ms.mean() * 1e3:.1f} us; "
        f"{achieved:.0f} GB/s algorithmic")

    result = {
        "metric": "paged decode attention achieved HBM GB/s (% of peak); decode tokens/s per layer",
        "value": round(tokens_per_s, 1),
        "unit": "decode tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 kv, fp16 q/o, fp32 accumulate" if fp8 else "fp16",
        "data": "synthetic",
        "config": {
            "workload": f"config {args.config} ({w.name}): B={w.batch}, {w.n_q}/{w.n_kv} heads, "
                        f"head_dim {w.d}, block 16, pool {w.num_blocks} blocks scattered (+{extra} spare), "
                        f"split-K partition {args.partition} + reduce"
                        + (f", FP8 E4M3 KV pools (scales {FP8_K_SCALE:.6g}, {FP8_V_SCALE:.6g})"
                           if fp8 else ""),
            "kv_dtype": args.kv_dtype,
            "batch": w.batch,
            "mean_context": round(float(np.mean(stepper.last_lens)), 1),
            "partition": args.partition,
            "clock_warmup_ms": args.warm_ms,
            "flush_mb_between_steps": args.flush_mb,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": recorded_traffic(args.kv_dtype),
            "kernel": ("pa_paged_attention_decode_fp8" if fp8 else "pa_paged_attention_decode")
                      + " (decode_worklist_kernel + decode_reduce_kernel)",
            "algorithmic_bytes_per_launch": int(dec_bytes),
            "launch_us_mean": round(float(dec_ms.mean()) * 1e3, 2),
            "launch_us_p50": round(float(np.median(dec_ms)) * 1e3, 2),
            "launch_us_p99": round(float(np.percentile(dec_ms, 99)) * 1e3, 2),
            "reshape_and_cache_us_mean": round(float(cache_ms.mean()) * 1e3, 2),
            "kernel_source_sha256": kernel_source_hash(),
        },
        "cpu_baseline": None,
    }
    del cache, stepper
    torch.cuda.empty_cache()
    if not args.no_prefill:
        # the chunked-prefill part of the path, on the long-context workload:
        # compute-bound, so it is reported against the MFMA peak
        pms, pwall, pflops, pw = measure_prefill(args, args.kv_dtype)
        result["prefill"] = {
            "metric": "paged prefill chunk attention TFLOP/s (% of fp16 MFMA peak)",
            "value": round(pflops * len(pms) / pwall / 1e12, 2),
            "unit": "TFLOP/s",
            "steps": len(pms),
            "workload": prefill_workload_text(pw),
            "roofline": prefill_roofline(pms, pflops, args.kv_dtype),
            "cpu_baseline": None,
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_budget, total_steps, args.kv_dtype)
        if not args.no_prefill:
            del w
            result["prefill"]["cpu_baseline"] = cpu_prefill_baseline(pw, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
