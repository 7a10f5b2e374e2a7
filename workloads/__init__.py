"""Seeded synthetic inputs for paged attention over a block-tabled KV cache.

This package only draws inputs: block pools, block tables, context lengths,
query rows, new K/V rows and their slots.  It performs none of the attention
arithmetic.  Both the CPU oracle (through the tests) and the GPU library
consume what it returns; neither is imported here.
"""

from .synth import (  # noqa: F401
    PagedStep,
    make_decode_step,
    make_mixed_step,
    make_prefill_step,
    config_1,
    config_2,
    config_3,
    config_4,
    config_5,
    fused_qkv,
    CONFIG_NAMES,
)
from .accounting import decode_bytes, kv_write_bytes, prefill_bytes, prefill_flops, rope_kv_write_bytes  # noqa: F401
