"""CPU fp64 oracle for the paged-attention decode step (test infrastructure only).

Only tests, the smoke check and the bench's CPU-baseline leg import this package.
The HIP library never does, and nothing here calls into it.
"""

from .paged_decode import (  # noqa: F401
    bf16_bits_to_f64,
    cache_write,
    decode_step,
    gather_context,
    merge_partitions,
    paged_attention_decode,
    partition_stats,
    partitioned_attention_decode,
    slot_mapping,
    softmax_attention,
    to_f64,
    token_place,
)
