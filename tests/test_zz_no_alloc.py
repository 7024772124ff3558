"""pa_paged_attention_decode_noalloc (for callers that cannot allocate):
the decode partials live in the library's per-GPU scratch array instead of
a caller workspace.  Through the C ABI, its outputs must equal those of
pa_paged_attention_decode on the same inputs bit for bit (the same kernels
run), on two calls in a row, the second with a smaller input (the array
keeps the first call's contents), in both launch forms; inputs whose
partials exceed the array are refused before any launch."""
import numpy as np
import pytest
import torch

from gpu_util import gpu_run, log
from synth import make_tiny_workload, make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def noalloc(plan, q, worklist=True):
    import pagedattention_block_paged_reshape_amd as pa
    out = torch.full_like(plan.out, 9.0)
    pa.pa_paged_attention_decode_noalloc(
        out, q, plan.cache.kv, plan.tables, plan.max_blocks, plan.lens, plan.batch, plan.n_q,
        plan.scale, plan.partition, plan.max_len, plan.items if worklist else None,
        plan.n_items if worklist else 0, flags=plan.flags)
    return out


def test_noalloc_decode_equals_workspace_decode_on_two_calls():
    import pagedattention_block_paged_reshape_amd as pa
    from pagedattention_block_paged_reshape_amd import _lib as L
    from pagedattention_block_paged_reshape_amd.cache import DecodePlan
    # first call: the Llama-3-70B-shaped batch (34.6 MB of partials)
    w = make_workload(3)
    res = gpu_run(w, partition=512)
    plan, q = res["plan"], res["q"]
    need = pa.pa_decode_workspace_bytes(plan.batch, plan.n_q, w.d, plan.max_len, 512)
    assert 0 < need <= pa.PA_DECODE_SCRATCH_BYTES
    a = noalloc(plan, q)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), res["decode"].view(torch.int16))
    grid = DecodePlan(res["cache"], w.decode_ids, w.n_q, w.scale, 512, worklist=False)
    g = noalloc(grid, q, worklist=False)
    torch.cuda.synchronize()
    assert torch.equal(g.view(torch.int16), res["decode"].view(torch.int16))
    log(f"noalloc call 1: B={plan.batch}, {need} bytes of partials, bitwise equal")
    del res, plan, grid, a, g
    torch.cuda.empty_cache()
    # second call: a smaller batch with another head shape and partition size
    w2 = make_tiny_workload([3, 40, 700, 1300, 2049], n_q=16, n_kv=4, d=128, seed=81,
                            dist="normal")
    res2 = gpu_run(w2, partition=256)
    plan2 = res2["plan"]
    need2 = pa.pa_decode_workspace_bytes(plan2.batch, plan2.n_q, w2.d, plan2.max_len, 256)
    assert 0 < need2 < need
    b = noalloc(plan2, res2["q"])
    torch.cuda.synchronize()
    assert torch.equal(b.view(torch.int16), res2["decode"].view(torch.int16))
    log(f"noalloc call 2: B={plan2.batch}, {need2} bytes of partials, bitwise equal")
    # partials beyond the array: refused (PA_ERR_CAPACITY) before any launch
    too_long = int(np.ceil(pa.PA_DECODE_SCRATCH_BYTES / (plan2.batch * plan2.n_q * (2 * 128 + 8)))
                   * 256) + 256
    with pytest.raises(pa.PaError) as e:
        pa.pa_paged_attention_decode_noalloc(
            b, res2["q"], plan2.cache.kv, plan2.tables, too_long // 16, plan2.lens, plan2.batch,
            plan2.n_q, plan2.scale, 256, too_long, plan2.items, plan2.n_items)
    assert e.value.status == L.PA_ERR_CAPACITY
    again = noalloc(plan2, res2["q"])
    torch.cuda.synchronize()
    assert torch.equal(again.view(torch.int16), res2["decode"].view(torch.int16))
