"""Seeded synthetic decode batches shared by the tests, the bench and the smoke check.

This package only draws inputs (context lengths, block tables, Q/K/V values, poison
fill).  It holds none of the decode method's arithmetic: no slot computation, no
gather, no attention.  Both the HIP path and the CPU oracle consume what it makes.
"""

from .decode_batches import (  # noqa: F401
    CONFIGS,
    FP8_CONFIGS,
    MULTI_CONFIGS,
    PARTITION_BALANCED,
    DecodeBatch,
    build_batch,
    build_fp8_batch,
    build_multi_batch,
    make_config,
    make_fp8_config,
    make_multi_config,
    permute_physical_blocks,
    poison_bits,
    unshare_prefix_blocks,
)
