"""fp64 CPU oracle for paged attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the
C-ABI library and its Python binding) never calls it and shares no code with
it: the oracle has its own block-allocator model, its own model of the paged
K/V pool, and textbook softmax attention over the logically gathered sequence.

Sources (web pages on vLLM / PagedAttention; cited by page title and section):
  * ngrok summary "Serving models at scale with vLLM" (techfeed.io):
    "PagedAttention" section -- 16-token blocks, allocate when a block fills,
    blocks anywhere, block table; scheduler section -- preemption, chunked prefill.
  * "vLLM and PagedAttention" (media.tcdigital.jp): "logical/physical block
    mapping" and "memory sharing for parallel sampling" (copy-on-write).
  * "LLM serving from scratch" (ta-paperlens): prefill/decode, eq. (1), the
    KV-size example, "fragmentation and PagedAttention", FIG 1, the scheduler
    sketch.
  * "vLLM inference optimization" (youngju.dev): KV-cache size function,
    contiguous-waste example, PagedAttention manager, copy-on-write prefix
    sharing.
  * ngrok summary, "prefix caching" section: blocks shared by hash chain of
    the token prefix (oracle/prefix_cache.py); scheduler section and
    ta-paperlens "scheduler skeleton": continuous batching with decode
    first, chunked prefill and preemption (oracle/scheduler.py).
  * ta-paperlens "in practice" (KV-cache dtype as a setting): the FP8 E4M3
    codec of the FP8 KV-cache variant (oracle/fp8.py).

Every function is pinned by tests/test_oracle_*.py against values the pages
print, closed forms, library routines (torch CPU fp64 SDPA) and brute force.
No part of it is "parity unpinned".
"""
from .allocator import BlockPoolModel, OutOfBlocks  # noqa: F401
from .prefix_cache import PrefixCachingPoolModel  # noqa: F401
from .scheduler import SchedulerModel  # noqa: F401
from . import fp8  # noqa: F401
from .pool import Fp8PoolModel, PoolModel  # noqa: F401
from .attention import (  # noqa: F401
    decode_attention,
    decode_attention_one,
    prefill_chunk_attention,
    kv_bytes_per_token,
    kv_cache_size_gib,
    contiguous_waste,
    paged_waste,
)
from .replay import (  # noqa: F401
    OracleState,
    run_setup,
    run_step,
    decode_reference,
    prefill_reference,
)
