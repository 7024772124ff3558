"""GPU parity of the FP8 KV-cache variant (E4M3 codes, one scale per pool).

Stores are compared code for code with the oracle's E4M3 encoder, over every
fp16 bit pattern and several scales.  Attention over FP8 pools is compared
with the fp64 oracle attending the values the codes stand for (code value
times scale), at the fp16 path's tolerance: the kernel widens the codes to
fp16 exactly, so the only differences left are those of the fp16 path
(fp16 probabilities, fp32 accumulation, fp16 output).  How far FP8 outputs lie
from the unquantised fp16 ones is logged, not tested: the pages fix no format
and so no accuracy."""
import numpy as np
import pytest
import torch

from gpu_util import (FILL8, assert_close, assert_pools_bit_exact, gpu_run, log, oracle_run,
                      shared_oracle, shared_reference, shared_workload,
                      pools8_to_logical)
from oracle import decode_reference, prefill_reference
from oracle.fp8 import decode_e4m3
from oracle.pool import Fp8PoolModel
from synth import make_mixed_workload, make_tiny_workload, make_workload

pytestmark = pytest.mark.gpu

RAGGED = [1, 15, 16, 17, 100, 511, 512, 513, 1000, 2047]
# per-pool scales of N(0, 1) rows: about max |x| / 448, deliberately not powers of two
K_SCALE, V_SCALE = 5.5 / 448, 4.75 / 448


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ stores

@pytest.mark.parametrize("k_scale,v_scale", [(1.0, 1.0), (0.0123, 1000.0), (3.0, 2.0 ** -10)])
def test_store_quantises_every_fp16_value(k_scale, v_scale):
    """256 tokens x 2 heads x 128 dims hold all 65,536 fp16 bit patterns (K in
    order, V reversed), stored to scattered slots; two more tokens carry a
    negative and an out-of-range slot and must not be stored."""
    import pagedattention_block_paged_reshape_amd as pa
    from pagedattention_block_paged_reshape_amd.cache import PagedKVCache
    n_kv, d, nb = 2, 128, 20
    bits = np.arange(65536, dtype=np.uint16)
    k = bits.view(np.float16).reshape(256, n_kv, d)
    v = bits[::-1].copy().view(np.float16).reshape(256, n_kv, d)
    rng = np.random.default_rng(41)
    slots = rng.permutation(nb * 16)[:256].astype(np.int32)
    extra = np.zeros((2, n_kv, d), dtype=np.float16)
    k_all, v_all = np.concatenate([k, extra]), np.concatenate([v, extra])
    slots_all = np.concatenate([slots, [-1, nb * 16 + 3]]).astype(np.int32)
    log(f"[fp8 store] scales ({k_scale}, {v_scale})")
    cache = PagedKVCache(nb, n_kv, d, device="cuda:0", fill_byte=FILL8, kv_dtype="fp8",
                         k_scale=k_scale, v_scale=v_scale)
    dk, dv = torch.from_numpy(k_all).cuda(), torch.from_numpy(v_all).cuda()
    pa.pa_reshape_and_cache_fp8(dk, dv, torch.from_numpy(slots_all).cuda(), len(slots_all),
                                cache.kv)
    torch.cuda.synchronize()
    ref = Fp8PoolModel(nb, n_kv, d, k_scale, v_scale)
    ref.write(k, v, slots)
    kd, vd = pools8_to_logical(cache.k_pool.cpu().numpy(), cache.v_pool.cpu().numpy(), d)
    kd, vd = kd.transpose(0, 2, 1, 3), vd.transpose(0, 2, 1, 3)          # [N][16][H][d]
    blk, off = slots // 16, slots % 16
    for got, want, rows in ((kd[blk, off], ref.k.transpose(0, 2, 1, 3)[blk, off], k),
                            (vd[blk, off], ref.v.transpose(0, 2, 1, 3)[blk, off], v)):
        nan_in = np.isnan(rows.astype(np.float32))
        # a NaN input may keep its sign: both E4M3 NaN codes are accepted
        assert np.isin(got[nan_in], [0x7F, 0xFF]).all()
        bad = (got != want) & ~nan_in
        assert not bad.any(), (f"{bad.sum()} codes differ; first input "
                               f"{rows[bad][0]!r}: got {got[bad][0]:#04x} want {want[bad][0]:#04x}")
    unused = np.ones(nb * 16, dtype=bool)
    unused[slots] = False
    kraw = cache.k_pool.cpu().numpy()
    assert (kd.reshape(nb * 16, -1)[unused] == FILL8).all()
    assert (vd.reshape(nb * 16, -1)[unused] == FILL8).all()
    assert kraw.size == nb * n_kv * 16 * d
    finite = ~np.isnan(decode_e4m3(kd[blk, off]))
    assert finite.sum() == (~np.isnan(k.astype(np.float32))).sum()
    cache.close()


@pytest.mark.parametrize("cfg", ["1", "4", "4b"])
def test_fp8_config_cache_and_decode(cfg):
    """A whole step over FP8 pools: slots, copy-on-write copies (4b: 127 of
    them) and every stored code equal the oracle's; decode within tolerance."""
    w = make_workload(cfg)
    ks, vs = (1.0 / 448, 1.0 / 448) if cfg == "1" else (K_SCALE, V_SCALE)
    st = oracle_run(w, "fp8", ks, vs)
    res = gpu_run(w, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    assert res["step_slots"].tolist() == st.step_slots.tolist()
    assert [tuple(c) for c in res["step_copies"].tolist()] == st.step_copies
    n = assert_pools_bit_exact(res["cache"], st)
    err = assert_close(res["decode"], decode_reference(w, st), f"fp8 config {cfg} decode")
    log(f"fp8 config {cfg}: {n} live slots code-exact, decode max err {err:.2e}")


def test_fp8_config3_full_size_decode():
    """The FP8 decode workload the benchmark times (the Llama-3-70B-shaped
    batch): every stored code, and every output element (all 256 requests,
    heads and dims) against the oracle; the grid form, KEEP loads and a second
    launch give bitwise the same result.  Also logs the distance to the
    unquantised fp16 result."""
    from pagedattention_block_paged_reshape_amd.cache import DecodePlan
    w = shared_workload(3)
    st = shared_oracle(3, "fp8", K_SCALE, V_SCALE)
    res = gpu_run(w, partition=512, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    n = assert_pools_bit_exact(res["cache"], st)
    ref = shared_reference(3, "decode", "fp8", K_SCALE, V_SCALE)
    err = assert_close(res["decode"], ref, "fp8 config 3 decode (all 256 requests)")
    grid = DecodePlan(res["cache"], w.decode_ids, w.n_q, w.scale, 512, worklist=False)
    keep = DecodePlan(res["cache"], w.decode_ids, w.n_q, w.scale, 512, keep_kv=True)
    g_out = grid.run(res["q"]).clone()
    k_out = keep.run(res["q"]).clone()
    again = res["plan"].run(res["q"]).clone()
    torch.cuda.synchronize()
    for other in (g_out, k_out, again):
        assert torch.equal(other.view(torch.int16), res["decode"].view(torch.int16))
    exact = decode_reference(w, shared_oracle(3), seq_index=range(0, w.batch, 16))
    got = res["decode"].float().cpu().numpy()[::16]
    log(f"fp8 config 3: {n} live slots code-exact, max err vs oracle {err:.2e}; vs unquantised "
        f"fp16 K/V: max {np.abs(got - exact).max():.3e}, mean {np.abs(got - exact).mean():.3e}")


@pytest.mark.parametrize("worklist", [True, False])
@pytest.mark.parametrize("partition", [16, 48, 512, 4096])
def test_fp8_decode_partition_sizes(partition, worklist):
    w = make_tiny_workload(RAGGED, n_q=32, n_kv=8, d=128, seed=23, dist="normal")
    st = oracle_run(w, "fp8", K_SCALE, V_SCALE)
    res = gpu_run(w, partition=partition, worklist=worklist, kv_dtype="fp8", k_scale=K_SCALE,
                  v_scale=V_SCALE)
    assert_close(res["decode"], decode_reference(w, st), f"fp8 partition {partition}")


@pytest.mark.parametrize("n_q,n_kv,d", [(16, 1, 128), (8, 8, 64), (4, 2, 64), (12, 4, 128),
                                        (16, 4, 64)])
def test_fp8_decode_head_shapes(n_q, n_kv, d):
    w = make_tiny_workload([1, 17, 64, 300, 700], n_q=n_q, n_kv=n_kv, d=d, seed=n_q * 5 + d,
                           dist="normal")
    st = oracle_run(w, "fp8", K_SCALE, V_SCALE)
    res = gpu_run(w, partition=256, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    assert_close(res["decode"], decode_reference(w, st), f"fp8 heads {n_q}/{n_kv} d{d}")


def test_fp8_decode_with_saturated_codes():
    """Scales too small for the data: many codes saturate at +-448; the
    kernel still attends exactly the values the codes stand for."""
    w = make_tiny_workload(RAGGED, n_q=16, n_kv=2, d=128, seed=29, dist="normal")
    ks, vs = 1.0 / 448, 0.5 / 448
    st = oracle_run(w, "fp8", ks, vs)
    res = gpu_run(w, partition=512, kv_dtype="fp8", k_scale=ks, v_scale=vs)
    assert_pools_bit_exact(res["cache"], st)
    codes = res["cache"].k_pool.cpu().numpy()
    assert np.isin(codes, [0x7E, 0xFE]).mean() > 0.05
    assert_close(res["decode"], decode_reference(w, st), "fp8 saturated")


def test_fp8_decode_is_placement_invariant():
    w = make_tiny_workload(RAGGED, n_q=32, n_kv=8, d=128, seed=31, dist="normal")
    a = gpu_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    w.free_order = np.random.default_rng(77).permutation(w.num_blocks).astype(np.int32)
    b = gpu_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a["decode"].view(torch.int16), b["decode"].view(torch.int16))


# --------------------------------------------------------------- prefill

@pytest.mark.parametrize("decode_lengths,q_start,chunk,n_q,n_kv,d", [
    ([], 0, 48, 4, 2, 128),            # whole causal prompt from position 0
    ([17, 300], 37, 100, 32, 8, 128),  # unaligned start, ragged end, decode beside it
    ([], 640, 129, 16, 16, 128),       # G = 1
    ([], 333, 77, 64, 8, 128),         # G = 8
    ([], 250, 130, 8, 2, 64),          # head_dim 64
    ([], 4093, 512, 32, 8, 128),       # several key splits
])
def test_fp8_prefill_chunk_parity(decode_lengths, q_start, chunk, n_q, n_kv, d):
    """Causal chunks over FP8 pools (every pool byte starts as a NaN code, so
    an unmasked code past the end shows): within tolerance of the oracle
    attending the dequantised values."""
    w = make_mixed_workload(decode_lengths, q_start, chunk, n_q=n_q, n_kv=n_kv, d=d,
                            seed=5 * q_start + chunk)
    st = oracle_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    res = gpu_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    assert_pools_bit_exact(res["cache"], st)
    err = assert_close(res["prefill"], prefill_reference(w, st), "fp8 prefill")
    if w.batch:
        assert_close(res["decode"], decode_reference(w, st), "fp8 decode beside the chunk")
    log(f"fp8 prefill q_start={q_start} chunk={chunk} G={n_q // n_kv} d={d}: max err {err:.2e}")


def test_fp8_config5_prefill_chunk():
    """The long-context chunk (512 rows at 49,488) over FP8 pools, in the
    launch the fp16 bench times; every row, head and dim."""
    w = shared_workload(5)
    res = gpu_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE, decode=False)
    err = assert_close(res["prefill"], shared_reference(5, "prefill", "fp8", K_SCALE, V_SCALE),
                       "fp8 config 5 prefill (all 512 rows x 32 heads)")
    log(f"fp8 config 5 prefill: max err {err:.2e}")


# ------------------------------------------------------------ mixed launch

def _run_mixed_fp8(w, res, partition=512, keep_kv=None):
    from pagedattention_block_paged_reshape_amd.cache import MixedPlan
    pf = w.prefill
    plan = MixedPlan(res["cache"], w.decode_ids, pf.seq_id, pf.q_start, pf.chunk_len, w.n_q,
                     w.scale, partition, keep_kv=keep_kv)
    dev = res["cache"].device
    d_out, p_out = plan.run(torch.from_numpy(w.q).to(dev), torch.from_numpy(pf.q).to(dev))
    torch.cuda.synchronize()
    return plan, d_out.clone(), p_out.clone()


@pytest.mark.parametrize("decode_lengths,q_start,chunk,n_q,n_kv,d,keep", [
    ([5, 16, 17, 33], 0, 48, 4, 2, 128, False),        # tiny decode + whole causal prompt
    ([1, 600, 1537, 2049], 37, 100, 32, 8, 128, False),  # multi-partition decode, ragged chunk
    ([90, 1025], 333, 77, 64, 8, 128, False),          # G = 8
    ([300, 45, 1100], 250, 130, 8, 2, 64, False),      # head_dim 64
    ([4096, 3, 129], 4093, 512, 32, 8, 128, False),    # several key splits
    ([40, 300], 200, 64, 32, 8, 128, True),            # KEEP decode loads
])
def test_fp8_mixed_equals_separate_launches_and_oracle(decode_lengths, q_start, chunk, n_q,
                                                        n_kv, d, keep):
    """pa_paged_attention_mixed_fp8: bitwise the FP8 decode and prefill
    launches on the same pool, within tolerance of the oracle attending the
    dequantised values."""
    w = make_mixed_workload(decode_lengths, q_start, chunk, n_q=n_q, n_kv=n_kv, d=d,
                            seed=3 * q_start + chunk + 1)
    st = oracle_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    res = gpu_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE, keep_kv=keep or None)
    _, d_out, p_out = _run_mixed_fp8(w, res, keep_kv=keep or None)
    assert torch.equal(d_out.view(torch.int16), res["decode"].view(torch.int16))
    assert torch.equal(p_out.view(torch.int16), res["prefill"].view(torch.int16))
    err = assert_close(d_out, decode_reference(w, st), "fp8 mixed decode")
    errp = assert_close(p_out, prefill_reference(w, st), "fp8 mixed prefill")
    log(f"fp8 mixed {decode_lengths} q_start={q_start} chunk={chunk} d={d} keep={keep}: "
        f"decode {err:.2e}, prefill {errp:.2e}")


def test_fp8_mixed_many_units_per_walk():
    """One-block partitions: several decode units per wavefront pair in the
    FP8 mixed launch (two pairs per workgroup, pairs of one workgroup with
    different unit counts), bitwise the separate FP8 launches."""
    w = make_mixed_workload([8000, 6000, 3000, 900, 40, 2], 300, 64, n_q=32, n_kv=8, d=128,
                            seed=91)
    st = oracle_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    res = gpu_run(w, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE, partition=16)
    _, d_out, p_out = _run_mixed_fp8(w, res, partition=16)
    assert torch.equal(d_out.view(torch.int16), res["decode"].view(torch.int16))
    assert torch.equal(p_out.view(torch.int16), res["prefill"].view(torch.int16))
    err = assert_close(d_out, decode_reference(w, st), "fp8 mixed decode, one-block partitions")
    assert_close(p_out, prefill_reference(w, st), "fp8 mixed prefill")
    log(f"fp8 mixed, one-block partitions: decode {err:.2e}")


def test_fp8_config5_mixed_launch_and_scale_checks():
    """The long-context step over FP8 pools at full size: bitwise the separate
    FP8 launches; both outputs against the oracle in full.  Non-positive or
    non-finite scales are refused before any launch."""
    import pagedattention_block_paged_reshape_amd as pa
    from pagedattention_block_paged_reshape_amd import _lib as L
    w = shared_workload(5)
    res = gpu_run(w, partition=512, kv_dtype="fp8", k_scale=K_SCALE, v_scale=V_SCALE)
    plan, d_out, p_out = _run_mixed_fp8(w, res)
    assert torch.equal(d_out.view(torch.int16), res["decode"].view(torch.int16))
    assert torch.equal(p_out.view(torch.int16), res["prefill"].view(torch.int16))
    err = assert_close(d_out, shared_reference(5, "decode", "fp8", K_SCALE, V_SCALE),
                       "fp8 config 5 mixed decode")
    errp = assert_close(p_out, shared_reference(5, "prefill", "fp8", K_SCALE, V_SCALE),
                        "fp8 config 5 mixed prefill (all 512 rows x 32 heads)")
    kv = res["cache"].kv
    for ks, vs in [(0.0, 1.0), (1.0, -1.0), (float("inf"), 1.0), (1.0, float("nan"))]:
        bad = L.pa_kv_view_fp8(kv.k_pool, kv.v_pool, kv.num_blocks, kv.block_size,
                               kv.num_kv_heads, kv.head_dim, ks, vs)
        with pytest.raises(pa.PaError):
            pa.pa_paged_attention_mixed(plan.c_dec, plan.c_pf, bad, w.n_q, w.scale,
                                        plan.workspace, plan.ws_bytes)
    log(f"fp8 config 5 mixed: decode max err {err:.2e}, prefill max err {errp:.2e}")
