"""GPU parity of the mixed launch (pa_paged_attention_mixed): the decode
requests and the prefill chunk of one step computed by one kernel, then one
merge kernel.

Its outputs must equal, bit for bit, those of the separate decode and prefill
launches on the same pool (the same arithmetic in the same order), and the
fp64 oracle within |gpu - oracle| <= 2e-3 + 1e-2 * |oracle|."""
import numpy as np
import pytest
import torch

from gpu_util import assert_close, gpu_run, log, oracle_run, shared_reference, shared_workload
from oracle import decode_reference, prefill_reference
from synth import make_mixed_workload, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def run_mixed(w, res, partition=512, keep_kv=None):
    from pagedattention_block_paged_reshape_amd.cache import MixedPlan
    pf = w.prefill
    plan = MixedPlan(res["cache"], w.decode_ids, pf.seq_id, pf.q_start, pf.chunk_len, w.n_q,
                     w.scale, partition, keep_kv=keep_kv)
    q = torch.from_numpy(w.q).to(res["cache"].device)
    qc = torch.from_numpy(pf.q).to(res["cache"].device)
    d_out, p_out = plan.run(q, qc)
    torch.cuda.synchronize()
    return plan, d_out.clone(), p_out.clone()


def bitwise_equal(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("decode_lengths,q_start,chunk,n_q,n_kv,d,partition", [
    ([5, 16, 17, 33], 0, 48, 4, 2, 128, 512),         # tiny decode + whole causal prompt
    ([1, 600, 1537, 2049], 37, 100, 32, 8, 128, 512),  # multi-partition decode, ragged chunk
    ([513, 31, 4000], 1000, 300, 32, 8, 128, 256),     # split prefill rows, partition 256
    ([700, 12], 640, 129, 16, 16, 128, 512),           # G = 1
    ([90, 1025], 333, 77, 64, 8, 128, 512),            # G = 8
    ([2000], 90, 50, 16, 1, 128, 512),                 # G = 16
    ([300, 45, 1100], 250, 130, 8, 2, 64, 512),        # head_dim 64
    ([4096, 3, 129], 4093, 512, 32, 8, 128, 512),      # several key splits
    # many units per decode walk (one-block partitions): several units per
    # wavefront pair, pairs of one workgroup with different unit counts
    ([8000, 6000, 3000, 900, 40, 2], 300, 64, 32, 8, 128, 16),
    # G = 16: three pairs per workgroup and a 2-unit result ring that wraps
    ([12000, 12000, 12000, 1000], 100, 64, 16, 1, 128, 16),
])
def test_mixed_equals_separate_launches_and_oracle(decode_lengths, q_start, chunk, n_q, n_kv,
                                                    d, partition):
    w = make_mixed_workload(decode_lengths, q_start, chunk, n_q=n_q, n_kv=n_kv, d=d,
                            seed=7 * q_start + chunk)
    st = oracle_run(w)
    res = gpu_run(w, partition=partition)
    _, d_out, p_out = run_mixed(w, res, partition)
    assert bitwise_equal(d_out, res["decode"]), "mixed decode differs from the decode launch"
    assert bitwise_equal(p_out, res["prefill"]), "mixed prefill differs from the prefill launch"
    err = assert_close(d_out, decode_reference(w, st), "mixed decode")
    errp = assert_close(p_out, prefill_reference(w, st), "mixed prefill")
    log(f"mixed {decode_lengths} q_start={q_start} chunk={chunk} G={n_q // n_kv} d={d}: "
        f"decode {err:.2e}, prefill {errp:.2e}")


def test_config5_mixed_launch():
    """The long-context step at full size: 8 decode requests at 32,768 tokens
    and the 512-row chunk at offset 49,488, in the launch configuration the
    mixed bench times.  Bitwise equal to the separate launches; both outputs
    against the oracle in full (every request, chunk row, head and dim)."""
    w = shared_workload(5)
    res = gpu_run(w, partition=512)
    plan, d_out, p_out = run_mixed(w, res)
    assert bitwise_equal(d_out, res["decode"])
    assert bitwise_equal(p_out, res["prefill"])
    err = assert_close(d_out, shared_reference(5, "decode"), "config 5 mixed decode")
    errp = assert_close(p_out, shared_reference(5, "prefill"),
                        "config 5 mixed prefill (all 512 rows x 32 heads)")
    # repeated launches on one workspace give the same bits
    q = torch.from_numpy(w.q).to(res["cache"].device)
    qc = torch.from_numpy(w.prefill.q).to(res["cache"].device)
    for _ in range(3):
        a, b = plan.run(q, qc)
    torch.cuda.synchronize()
    assert bitwise_equal(a, d_out) and bitwise_equal(b, p_out)
    log(f"config 5 mixed: decode max err {err:.2e}, prefill max err {errp:.2e}")


def test_mixed_keep_kv_loads():
    """Decode with PA_DECODE_KEEP_KV (cached K/V loads, the setting for
    batches that share blocks) next to a chunk of another request: bitwise
    the separate launches, within tolerance of the oracle."""
    w = make_mixed_workload([40, 300], 200, 64, n_q=32, n_kv=8, d=128, seed=11)
    st = oracle_run(w)
    res = gpu_run(w, keep_kv=True)
    _, d_out, p_out = run_mixed(w, res, keep_kv=True)
    assert bitwise_equal(d_out, res["decode"])
    assert bitwise_equal(p_out, res["prefill"])
    assert_close(d_out, decode_reference(w, st), "mixed decode, KEEP loads")
    assert_close(p_out, prefill_reference(w, st), "mixed prefill next to KEEP decode")


def test_mixed_with_one_part_empty():
    """An empty decode batch runs the chunk alone, an empty chunk the decode
    batch alone; outputs of the missing part are not touched."""
    import pagedattention_block_paged_reshape_amd as pa
    w = make_mixed_workload([70, 1300], 500, 90, n_q=32, n_kv=8, d=128, seed=4)
    st = oracle_run(w)
    res = gpu_run(w)
    plan, d_out, p_out = run_mixed(w, res)
    dev = res["cache"].device
    q = torch.from_numpy(w.q).to(dev)
    qc = torch.from_numpy(w.prefill.q).to(dev)
    d_sent = torch.full_like(d_out, 5.0)
    p_sent = torch.full_like(p_out, 6.0)
    d, p = plan.dec, plan.pf
    no_dec = pa.decode_batch(d_sent, q, d.tables, d.max_blocks, d.lens, 0, d.partition,
                             d.max_len, d.items, d.n_items)
    chunk = pa.prefill_chunk(p_sent, qc, p.table, p.table_len, p.q_start, p.chunk_len)
    pa.pa_paged_attention_mixed(no_dec, chunk, res["cache"].kv, w.n_q, w.scale, plan.workspace,
                                plan.ws_bytes)
    torch.cuda.synchronize()
    assert (d_sent.float() == 5.0).all()
    assert bitwise_equal(p_sent, p_out)
    d_sent.fill_(5.0)
    p_sent.fill_(6.0)
    dec = pa.decode_batch(d_sent, q, d.tables, d.max_blocks, d.lens, d.batch, d.partition,
                          d.max_len, d.items, d.n_items)
    no_chunk = pa.prefill_chunk(p_sent, qc, p.table, p.table_len, p.q_start, 0)
    pa.pa_paged_attention_mixed(dec, no_chunk, res["cache"].kv, w.n_q, w.scale, plan.workspace,
                                plan.ws_bytes)
    torch.cuda.synchronize()
    assert (p_sent.float() == 6.0).all()
    assert bitwise_equal(d_sent, d_out)
    assert_close(d_sent, decode_reference(w, st), "decode alone through the mixed launch")
    with pytest.raises(pa.PaError):          # n_q not a multiple of the kv heads
        pa.pa_paged_attention_mixed(dec, chunk, res["cache"].kv, w.n_q - 1, w.scale,
                                    plan.workspace, plan.ws_bytes)
    assert np.isfinite(d_out.float().cpu().numpy()).all()


def test_mixed_decode_give_up_writes_nan_not_stale_rows(monkeypatch):
    """The mixed launch's decode walks have the decode launch's bounded LDS
    slot wait.  With the bound forced to 0 rounds from the host (a test hook;
    every wait still ends) a wavefront that finds a slot still busy gives up:
    every decode row is then NaN or bitwise the normal run's, the chunk's rows
    are exact, and a normal launch afterwards is bitwise the separate
    launches again."""
    w = make_mixed_workload([8000, 6000, 3000, 900, 40, 2], 300, 64, n_q=32, n_kv=8, d=128,
                            seed=83)
    res = gpu_run(w, partition=16)
    plan, d_out, p_out = run_mixed(w, res, 16)
    assert bitwise_equal(d_out, res["decode"]) and bitwise_equal(p_out, res["prefill"])
    good = d_out.float().cpu().numpy()
    q = torch.from_numpy(w.q).to(res["cache"].device)
    qc = torch.from_numpy(w.prefill.q).to(res["cache"].device)
    monkeypatch.setenv("PA_DECODE_SPIN_LIMIT", "0")
    nan_rows = 0
    for rep in range(5):
        plan.dec.out.fill_(3.0)              # stale contents the give-up must not leave
        a, b = plan.run(q, qc)
        torch.cuda.synchronize()
        got = a.float().cpu().numpy()
        is_nan = np.isnan(got).all(axis=-1)
        same = (got.view(np.uint32) == good.view(np.uint32)).all(axis=-1)
        assert (is_nan | same).all(), "a decode row is neither NaN nor the normal result"
        assert bitwise_equal(b, p_out), "the chunk's rows changed"
        nan_rows += int(is_nan.sum())
    monkeypatch.delenv("PA_DECODE_SPIN_LIMIT")
    a, b = plan.run(q, qc)
    torch.cuda.synchronize()
    assert bitwise_equal(a, res["decode"]) and bitwise_equal(b, res["prefill"])
    log(f"mixed give-up: {nan_rows} of {5 * good.shape[0] * good.shape[1]} decode rows NaN "
        f"over 5 runs")
