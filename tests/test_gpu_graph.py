"""The attention launches captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the work-list decode with its reduce (caller workspace and the
no-allocation entry point), the prefill chunk with its split merge, and the
mixed launch.  None of them allocates, frees or clears memory inside the
captured region, so a graph of a step replays the same kernels on the same
buffers (a serving loop that replays a captured step: ta-paperlens,
scheduler skeleton).

Each graph is replayed several times with the program's own eager launches
and synchronisations in between; every replay must be bitwise the eager
result, which itself is checked against the fp64 oracle elsewhere."""
import pytest
import torch

from gpu_util import gpu_run, log, shared_workload
from synth import make_mixed_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def bitwise_equal(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def replay_and_check(name, launch, outs, expected, between, reps=4):
    """Capture launch(stream) once, then replay it `reps` times: before each
    replay the outputs are poisoned and `between()` runs eager work; after
    it every output must equal its expected tensor bit for bit."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        launch(side)                            # warm-up off the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        launch(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for rep in range(reps):
        for o in outs:
            o.fill_(float("nan"))
        between()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, expected):
            assert bitwise_equal(o, e), f"{name}: replay {rep} differs from the eager launch"
    log(f"[graph] {name}: {reps} replays bitwise equal to the eager launch")
    del graph


def test_decode_replays_from_a_graph():
    """Config 2 (64 requests, up to 4 partitions each): the work-list decode
    and its reduce, with the caller's workspace and through the
    no-allocation entry point."""
    import pagedattention_block_paged_reshape_amd as pa
    w = shared_workload("2")
    res = gpu_run(w, partition=512)
    plan, q, eager = res["plan"], res["q"], res["decode"]
    out = plan.out
    replay_and_check("decode", lambda s: plan.run(q, s), [out], [eager],
                     between=lambda: plan.run(q))

    na_out = torch.empty_like(out)

    def noalloc(s):
        pa.pa_paged_attention_decode_noalloc(
            na_out, q, plan.cache.kv, plan.tables, plan.max_blocks, plan.lens, plan.batch,
            plan.n_q, plan.scale, plan.partition, plan.max_len, plan.items, plan.n_items,
            flags=plan.flags, stream=s)

    noalloc(torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert bitwise_equal(na_out, eager)
    # between the replays: an eager no-allocation launch of another batch
    # overwrites the shared scratch array
    w2 = make_mixed_workload([3, 900, 2049], 0, 16, n_q=16, n_kv=4, d=128, seed=5)
    res2 = gpu_run(w2, partition=256)
    p2, q2 = res2["plan"], res2["q"]
    other = torch.empty_like(p2.out)

    def between():
        pa.pa_paged_attention_decode_noalloc(
            other, q2, p2.cache.kv, p2.tables, p2.max_blocks, p2.lens, p2.batch, p2.n_q,
            p2.scale, p2.partition, p2.max_len, p2.items, p2.n_items, flags=p2.flags)

    replay_and_check("decode, no-allocation entry", noalloc, [na_out], [eager], between)
    torch.cuda.synchronize()
    assert bitwise_equal(other, res2["decode"])


def test_prefill_and_mixed_replay_from_a_graph():
    """A chunk with several key splits (merged by the second kernel) next to
    a decode batch with long requests: the prefill launch alone and the
    mixed launch."""
    from pagedattention_block_paged_reshape_amd.cache import MixedPlan
    w = make_mixed_workload([4096, 3, 129, 1500], 4093, 512, n_q=32, n_kv=8, d=128, seed=13)
    res = gpu_run(w, partition=512)
    pp, qc = res["pplan"], res["qc"]
    replay_and_check("prefill", lambda s: pp.run(qc, s), [pp.out], [res["prefill"]],
                     between=lambda: pp.run(qc))
    pf = w.prefill
    mp = MixedPlan(res["cache"], w.decode_ids, pf.seq_id, pf.q_start, pf.chunk_len, w.n_q,
                   w.scale, 512)
    q = res["q"]
    d_out, p_out = mp.run(q, qc)
    torch.cuda.synchronize()
    assert bitwise_equal(d_out, res["decode"]) and bitwise_equal(p_out, res["prefill"])
    replay_and_check("mixed", lambda s: mp.run(q, qc, s), [mp.dec.out, mp.pf.out],
                     [res["decode"], res["prefill"]],
                     between=lambda: (mp.run(q, qc), pp.run(qc)))
