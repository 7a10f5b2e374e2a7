"""Algorithmic work per call: the bytes or FLOPs a call must move or do at
minimum, used to turn measured times into GB/s and TFLOP/s.

These are cost counts, not attention arithmetic; the figures are what each
kernel has to touch once:

* decode: every K and V row of every context token once, q in, out once,
  the block-table entries that cover the context, and the context lengths;
* KV write: each non-skipped new K and V row read once and written once, plus
  the slot indices;
* rotary KV write: the fused projection rows read once, rotated q written
  once, each non-skipped k and v row written once, positions and slots, and
  one table row (head_dim fp32) per distinct position;
* prefill: 4 * head_dim * num_q_heads FLOPs per (query row, visible key) pair
  (QK^T and PV, 2 FLOPs per multiply-add), counting only keys the causal mask
  keeps: a chunk of q rows after c cached tokens sees q*c + q*(q+1)/2 pairs.
"""

from __future__ import annotations

import torch


def _elt(dtype: torch.dtype) -> int:
    return torch.empty((), dtype=dtype).element_size()


def decode_bytes(step, seqs=None) -> int:
    """Minimum HBM bytes of one decode call over ``step``'s decode sequences."""
    e = _elt(step.dtype)
    ctx = step.decode_context_lens.to(torch.int64)
    if seqs is not None:
        ctx = ctx[seqs]
    S = int(ctx.numel())
    kv = int(ctx.sum()) * step.num_kv_heads * step.head_dim * 2 * e
    qo = 2 * S * step.num_q_heads * step.head_dim * e
    tables = int(((ctx + step.block_size - 1) // step.block_size).sum()) * 4
    return kv + qo + tables + 4 * S


def kv_write_bytes(step) -> int:
    """Minimum HBM bytes of one KV-cache write call."""
    if step.slot_mapping is None:
        return 0
    e = _elt(step.dtype)
    rows = int((step.slot_mapping >= 0).sum())
    row_bytes = step.num_kv_heads * step.head_dim * e
    return rows * row_bytes * 2 * 2 + 8 * int(step.slot_mapping.numel())


def rope_kv_write_bytes(step) -> int:
    """Minimum HBM bytes of one fused rotary + KV-cache write call."""
    e = _elt(step.dtype)
    T = int(step.slot_mapping.numel())
    D, Hq, Hkv = step.head_dim, step.num_q_heads, step.num_kv_heads
    rows = int((step.slot_mapping >= 0).sum())
    read = T * (Hq + 2 * Hkv) * D * e + 16 * T + int(torch.unique(step.positions).numel()) * D * 4
    write = T * Hq * D * e + rows * 2 * Hkv * D * e
    return read + write


def prefill_flops(step) -> int:
    """Algorithmic FLOPs of one prefill call (unmasked pairs only)."""
    qsl = step.query_start_loc.tolist()
    ctx = step.prefill_context_lens.tolist()
    pairs = 0
    for j in range(step.num_prefill):
        q = qsl[j + 1] - qsl[j]
        c = ctx[j] - q
        pairs += q * c + q * (q + 1) // 2
    return 4 * step.head_dim * step.num_q_heads * pairs


def prefill_bytes(step) -> int:
    """Minimum HBM bytes of one prefill call: each chunk's visible K/V once,
    its q rows in and its out rows out, tables and lengths."""
    e = _elt(step.dtype)
    ctx = step.prefill_context_lens.to(torch.int64)
    kv = int(ctx.sum()) * step.num_kv_heads * step.head_dim * 2 * e
    rows = step.num_prefill_rows
    qo = 2 * rows * step.num_q_heads * step.head_dim * e
    tables = int(((ctx + step.block_size - 1) // step.block_size).sum()) * 4
    return kv + qo + tables + 4 * (2 * step.num_prefill + 1)
