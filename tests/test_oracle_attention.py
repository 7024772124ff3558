"""Pins for the oracle's attention (CPU only).

The oracle's decode and prefill must agree with independent computations:
scalar brute-force loops, torch's CPU fp64 scaled_dot_product_attention (a
library routine; GQA by repeating KV heads), closed-form special cases, and
the invariants paging must preserve (paged == contiguous, placement
permutation, shared == private, chunking)."""
import math

import numpy as np
import pytest
import torch

from oracle import (decode_attention, decode_attention_one, decode_reference,
                    prefill_chunk_attention, prefill_reference, run_setup, run_step)
from synth import make_tiny_workload, make_workload


def brute_force_decode(q, k, v, scale):
    """Scalar loops: no max subtraction, no vectorisation, G = n_q / n_kv."""
    n_q, d = q.shape
    L, n_kv, _ = k.shape
    G = n_q // n_kv
    out = np.zeros((n_q, d))
    for h in range(n_q):
        g = h // G
        w = []
        for j in range(L):
            s = 0.0
            for c in range(d):
                s += float(q[h, c]) * float(k[j, g, c])
            w.append(math.exp(scale * s))
        z = sum(w)
        for c in range(d):
            acc = 0.0
            for j in range(L):
                acc += w[j] * float(v[j, g, c])
            out[h, c] = acc / z
    return out


def torch_sdpa(q, k, v, scale, causal_offset=None):
    """torch CPU fp64 SDPA. q [R][n_q][d], k/v [L][n_kv][d]."""
    qt = torch.from_numpy(q.astype(np.float64)).permute(1, 0, 2)       # [n_q][R][d]
    G = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(G, 0)
    mask = None
    if causal_offset is not None:
        R, L = q.shape[0], k.shape[0]
        mask = torch.arange(L)[None, :] <= (causal_offset + torch.arange(R))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt.contiguous(), vt.contiguous(),
                                                         attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2).numpy()


def test_decode_matches_brute_force_loops():
    rng = np.random.default_rng(5)
    for L, n_q, n_kv, d in [(5, 4, 2, 16), (17, 4, 1, 8), (33, 8, 8, 4), (3, 16, 2, 8)]:
        q = rng.uniform(-1, 1, (n_q, d)).astype(np.float16)
        k = rng.uniform(-1, 1, (L, n_kv, d)).astype(np.float16)
        v = rng.uniform(-1, 1, (L, n_kv, d)).astype(np.float16)
        ref = brute_force_decode(q, k, v, 0.3)
        got = decode_attention_one(q, k, v, 0.3)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_decode_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(6)
    for L, n_q, n_kv, d in [(1, 4, 2, 64), (40, 32, 8, 128), (100, 64, 8, 128), (7, 2, 2, 64)]:
        q = rng.standard_normal((n_q, d)).astype(np.float16)
        k = rng.standard_normal((L, n_kv, d)).astype(np.float16)
        v = rng.standard_normal((L, n_kv, d)).astype(np.float16)
        ref = torch_sdpa(q[None], k, v, 1 / math.sqrt(d))[0]
        np.testing.assert_allclose(decode_attention_one(q, k, v, 1 / math.sqrt(d)), ref,
                                   rtol=1e-12, atol=1e-12)


def test_decode_special_cases():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((8, 32)).astype(np.float16)
    v = rng.standard_normal((20, 2, 32)).astype(np.float16)
    # one key: the single weight is 1, the output is that value row exactly
    k1 = rng.standard_normal((1, 2, 32)).astype(np.float16)
    o = decode_attention_one(q, k1, v[:1], 0.5)
    for h in range(8):
        assert np.array_equal(o[h], v[0, h // 4].astype(np.float64))
    # all keys equal: uniform weights, output is the mean of V
    keq = np.repeat(k1, 20, axis=0)
    o = decode_attention_one(q, keq, v, 0.5)
    for h in range(8):
        np.testing.assert_allclose(o[h], v[:, h // 4].astype(np.float64).mean(0), rtol=0,
                                   atol=1e-14)
    # zero query: uniform weights as well
    k = rng.standard_normal((20, 2, 32)).astype(np.float16)
    o = decode_attention_one(np.zeros_like(q), k, v, 0.5)
    np.testing.assert_allclose(o[3], v[:, 0].astype(np.float64).mean(0), atol=1e-14)
    # a dominant key takes all the weight
    kd = k.copy()
    kd[11, 1] = (q[5].astype(np.float32) * 40).astype(np.float16)
    o = decode_attention_one(q, kd, v, 1.0)
    np.testing.assert_allclose(o[5], v[11, 1].astype(np.float64), atol=1e-9)


def _replayed(w):
    st = run_setup(w, bulk=False)
    run_step(w, st)
    return st


def _contiguous_rows(w):
    """Each request's logical K/V straight from the workload's draw order
    (no paging): setup rows in append order, then its step row."""
    ks, vs = [], []
    lengths = w.notes["lengths"]
    c = 0
    for i, L in enumerate(lengths):
        ks.append(np.concatenate([w.setup_k[c:c + L - 1], w.step_k[i:i + 1]]))
        vs.append(np.concatenate([w.setup_v[c:c + L - 1], w.step_v[i:i + 1]]))
        c += L - 1
    return ks, vs


def test_paged_equals_contiguous_tiny_config():
    w = make_workload(1)
    st = _replayed(w)
    ks, vs = _contiguous_rows(w)
    for i in range(w.batch):
        gk, gv = st.pool.gather(st.alloc.tables[i], st.alloc.lens[i])
        assert np.array_equal(gk.view(np.uint16), ks[i].view(np.uint16))
        assert np.array_equal(gv.view(np.uint16), vs[i].view(np.uint16))
    got = decode_reference(w, st)
    ref = decode_attention(w.q, ks, vs, w.scale)
    assert np.array_equal(got, ref)
    for i in range(w.batch):
        np.testing.assert_allclose(got[i], brute_force_decode(w.q[i], ks[i], vs[i], w.scale),
                                   rtol=1e-12, atol=1e-13)


def test_tiny_config_block_accounting():
    """Attended lengths {5,16,17,33}: 5 blocks hold the cached tokens, the
    step's appends at offset 0 (positions 16 and 32) take 2 more."""
    w = make_workload(1)
    st = run_setup(w, bulk=False)
    assert st.alloc.num_blocks - st.alloc.num_free() == 5
    run_step(w, st)
    assert st.alloc.num_blocks - st.alloc.num_free() == 7
    assert [x % 16 for x in st.step_slots] == [4, 15, 0, 0]
    assert st.step_copies == []
    st.alloc.check()


def test_output_invariant_under_physical_permutation():
    w = make_tiny_workload([1, 15, 16, 17, 40, 64, 65], n_q=8, n_kv=2, d=32, num_blocks=40,
                           seed=11)
    base = decode_reference(w, _replayed(w))
    for s in range(3):
        w.free_order = np.random.default_rng(100 + s).permutation(w.num_blocks).astype(np.int32)
        st = _replayed(w)
        assert np.array_equal(decode_reference(w, st), base)


def test_shared_prefix_equals_private_copies():
    w = make_workload("4b")
    # shrink to keep the CPU test quick: 6 requests over the same prefix bytes
    B = 6
    w.decode_ids = w.decode_ids[:B]
    w.step_ids = w.step_ids[:B]
    w.step_n_new = w.step_n_new[:B]
    w.step_k, w.step_v, w.q = w.step_k[:B], w.step_v[:B], w.q[:B]
    w.setup = [op for op in w.setup if op[0] != "fork" or op[2] < B]
    st = _replayed(w)
    assert len(st.step_copies) == B - 1
    shared = decode_reference(w, st)
    P = w.notes["prefix"]
    for i in range(B):
        k = np.concatenate([w.setup_k[:P], w.step_k[i:i + 1]])
        v = np.concatenate([w.setup_v[:P], w.step_v[i:i + 1]])
        assert np.array_equal(shared[i], decode_attention_one(w.q[i], k, v, w.scale))


def _chunk_inputs(seed, P0, C, n_q=4, n_kv=2, d=16):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((C, n_q, d)).astype(np.float16)
    k = rng.standard_normal((P0 + C, n_kv, d)).astype(np.float16)
    v = rng.standard_normal((P0 + C, n_kv, d)).astype(np.float16)
    return q, k, v


def test_prefill_from_zero_is_causal_sdpa():
    q, k, v = _chunk_inputs(1, 0, 48)
    got = prefill_chunk_attention(q, k, v, 0, 0.25)
    ref = torch_sdpa(q, k, v, 0.25, causal_offset=0)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_prefill_with_offset_matches_sdpa_and_decode():
    P0, C = 37, 20
    q, k, v = _chunk_inputs(2, P0, C)
    got = prefill_chunk_attention(q, k, v, P0, 0.25)
    np.testing.assert_allclose(got, torch_sdpa(q, k, v, 0.25, causal_offset=P0),
                               rtol=1e-12, atol=1e-12)
    # each row equals a decode over the first P0 + r + 1 keys
    for r in (0, 7, C - 1):
        dec = decode_attention_one(q[r], k[:P0 + r + 1], v[:P0 + r + 1], 0.25)
        np.testing.assert_allclose(got[r], dec, rtol=1e-13, atol=1e-14)


def test_prefill_chunking_invariance_and_row_subsets():
    P0, C = 16, 64
    q, k, v = _chunk_inputs(3, P0, C)
    whole = prefill_chunk_attention(q, k, v, P0, 0.3)
    first = prefill_chunk_attention(q[:32], k[:P0 + 32], v[:P0 + 32], P0, 0.3)
    second = prefill_chunk_attention(q[32:], k, v, P0 + 32, 0.3)
    np.testing.assert_allclose(np.concatenate([first, second]), whole, rtol=1e-13, atol=1e-14)
    sub = prefill_chunk_attention(q, k, v, P0, 0.3, rows=[5, 63], heads=[3, 0])
    np.testing.assert_allclose(sub[0, 0], whole[5, 3], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sub[1, 1], whole[63, 0], rtol=1e-13, atol=1e-14)


def test_prefill_reference_on_paged_chunk():
    """A small mixed workload: the chunk's rows are appended in the step and
    read back through the paged pool."""
    from synth.workloads import Workload, PrefillChunk
    rng = np.random.default_rng(9)
    n_q, n_kv, d, P0, C = 4, 2, 16, 48, 32
    nb = 12
    setup_k = rng.standard_normal((P0, n_kv, d)).astype(np.float16)
    setup_v = rng.standard_normal((P0, n_kv, d)).astype(np.float16)
    step_k = rng.standard_normal((C, n_kv, d)).astype(np.float16)
    step_v = rng.standard_normal((C, n_kv, d)).astype(np.float16)
    qc = rng.standard_normal((C, n_q, d)).astype(np.float16)
    w = Workload(name="t", n_q=n_q, n_kv=n_kv, d=d, scale=0.25, num_blocks=nb,
                 free_order=rng.permutation(nb).astype(np.int32),
                 setup=[("add", 0), ("append", [0], [P0])], setup_k=setup_k, setup_v=setup_v,
                 step_ids=np.array([0]), step_n_new=np.array([C], np.int32), step_k=step_k,
                 step_v=step_v, decode_ids=np.zeros(0, np.int64), q=np.zeros((0, n_q, d)),
                 prefill=PrefillChunk(0, P0, C, qc))
    st = _replayed(w)
    got = prefill_reference(w, st)
    k = np.concatenate([setup_k, step_k])
    v = np.concatenate([setup_v, step_v])
    np.testing.assert_allclose(got, torch_sdpa(qc, k, v, 0.25, causal_offset=P0),
                               rtol=1e-12, atol=1e-12)
