"""Paged KV attention for AMD Instinct MI355X (gfx950).

A thin Python face over libpka.so (C ABI in include/pka.h): KV-cache write,
paged decode (single pass, split-K with its partition reduce, and the
dispatcher over both) and
paged prefill over ragged, causally masked chunks.  Tensors are torch GPU
tensors; the work runs in hand-written HIP kernels.  There is no CPU path:
importing the package without the built library raises ImportError.
"""

from ._lib import (  # noqa: F401
    LIB_PATH,
    PARTITION_SIZE,
    BlockManager,
    CacheDesc,
    PkaError,
    Prepared,
    cache_desc,
    decode_choose_variant,
    device_cu_count,
    fused_rope_kv_write,
    kv_cache_write,
    paged_attn_decode,
    paged_attn_decode_append,
    paged_attn_decode_noalloc,
    paged_attn_decode_splitk,
    paged_attn_decode_v1,
    paged_attn_prefill,
    paged_attn_splitk_reduce,
    prefill_split_keys,
    prefill_workspace,
    prefill_workspace_bytes,
    rope_table,
    splitk_buffers,
    splitk_workspace,
    splitk_workspace_bytes,
    version,
)
