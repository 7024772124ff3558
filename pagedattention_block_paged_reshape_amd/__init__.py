"""MI355X (gfx950) paged attention: host block manager + HIP kernels behind a C ABI.

The functions re-exported here carry the names of the C entry points declared
in include/pa.h; ``cache`` strings them together for one decode/prefill step.
Importing this package loads ``libpagedattn.so`` and fails if it is missing.
"""
from ._lib import (  # noqa: F401
    BLOCK_SIZE,
    EXPORTED,
    LIB_PATH,
    PA_DECODE_KEEP_KV,
    OutOfBlocksError,
    PaError,
    kv_view,
    pa_append_slots,
    pa_block_tables,
    pa_can_append,
    pa_copy_blocks,
    pa_decode_work_items,
    pa_decode_workspace_bytes,
    pa_evictable_list,
    pa_free_list,
    pa_kv_bytes_per_token,
    pa_num_free_blocks,
    pa_paged_attention_decode,
    pa_paged_attention_prefill,
    pa_pool_check,
    pa_pool_create,
    pa_pool_destroy,
    pa_pool_get_stats,
    pa_prefill_workspace_bytes,
    pa_ref_count,
    pa_reshape_and_cache,
    pa_seq_add,
    pa_seq_add_cached,
    pa_seq_fork,
    pa_seq_free,
    pa_seq_register,
    pa_seq_table,
    status_string,
)
