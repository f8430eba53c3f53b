"""PagedAttention decode on AMD MI355X (gfx950): Python binding of libpagedkv.so.

The hot path (slot mapping, cache write, paged attention with a log-sum-exp
partition merge) runs in hand-written HIP kernels behind the C ABI of
include/pagedkv.h; this package only marshals torch tensors into that ABI.
"""

from ._lib import LIB_PATH, PkvError, load_library, status_string  # noqa: F401
from .ops import (  # noqa: F401
    PARTITION_BALANCED,
    PARTITION_DEFAULT,
    BlockPool,
    DecodeStep,
    alloc_workspace,
    copy_blocks,
    decode_prologue,
    decode_prologue_fp8,
    decode_step,
    kv_cache_write,
    kv_cache_write_fp8,
    multi_query_workspace_bytes,
    paged_attention_decode,
    paged_attention_decode_fp8,
    paged_attention_decode_noalloc,
    paged_attention_decode_per_head,
    paged_attention_partition,
    paged_attention_multi_query,
    paged_attention_partition_fp8,
    paged_attention_partition_per_head,
    paged_attention_plan,
    prefix_block_hashes,
    paged_attention_reduce,
    slot_mapping,
    slot_mapping_multi_query,
    workspace_bytes,
)
