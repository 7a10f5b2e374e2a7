"""CPU fp64 oracle for rotary position embedding fused into the KV-cache write.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import or call this module.  The GPU library never
calls it and shares no code, header, table or helper with it.

What it computes, and where the pages place it:

* mini_engine ("Features", Model) builds the Qwen3 decoder with RoPE; its
  "Where the remaining gap comes from" section lists RoPE among the separate
  eager kernels, and its "Roadmap" folds RoPE into the QKV split / KV-cache
  write.  miniserve's "Engine" flowchart orders the layer as fused qkv
  projection, RoPE, then an index_copy_ that puts each new token's K and V
  rows into its pool slot.
* So one step takes the fused projection output of T tokens, rows
  ``[q heads | k heads | v heads]``, rotates q and k by each token's position,
  returns the rotated q and scatters the rotated k and the unchanged v into
  their slots (negative slots are padding and skipped, as in the KV write).

The rotation itself is not spelled out in the pages.  Reading (listed again in
the design notes): the standard rotary embedding over the whole head
dimension D, with the "rotate-half" pairing used by the Qwen model family:
element i < D/2 is paired with element i + D/2, and the pair is rotated by
the angle ``pos * theta ** (-2 i / D)``:

    out[i]       = x[i] cos(a_i) - x[i + D/2] sin(a_i)
    out[i + D/2] = x[i + D/2] cos(a_i) + x[i] sin(a_i)

theta is an argument (Qwen3 checkpoints use 1,000,000; the pages do not state
it).  Everything is computed in float64 from the exactly widened inputs and
rounded once to the input type at the end.
"""

from __future__ import annotations

import torch

__all__ = ["rope_angles", "rope", "split_qkv", "fused_rope_kv_write"]


def rope_angles(positions, head_dim: int, theta: float) -> torch.Tensor:
    """angle[t, i] = positions[t] * theta ** (-2 i / head_dim), i < head_dim / 2 (float64)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    half = head_dim // 2
    pos = torch.as_tensor(positions).to(torch.float64).reshape(-1, 1)
    inv_freq = torch.tensor([theta ** (-2.0 * i / head_dim) for i in range(half)], dtype=torch.float64)
    return pos * inv_freq.reshape(1, -1)


def rope(x: torch.Tensor, positions, theta: float) -> torch.Tensor:
    """Rotate x [T, H, D] (any float dtype) by each token's position; returns float64."""
    x = x.to(torch.float64)
    T, H, D = x.shape
    half = D // 2
    ang = rope_angles(positions, D, theta)  # [T, half]
    c = torch.cos(ang).reshape(T, 1, half)
    s = torch.sin(ang).reshape(T, 1, half)
    lo, hi = x[..., :half], x[..., half:]
    return torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1)


def split_qkv(qkv: torch.Tensor, num_q_heads: int, num_kv_heads: int):
    """Views of the fused projection rows [T, (Hq + 2 Hkv) * D] as q [T, Hq, D],
    k [T, Hkv, D], v [T, Hkv, D]."""
    T = qkv.shape[0]
    D = qkv.shape[1] // (num_q_heads + 2 * num_kv_heads)
    rows = qkv.reshape(T, num_q_heads + 2 * num_kv_heads, D)
    return rows[:, :num_q_heads], rows[:, num_q_heads:num_q_heads + num_kv_heads], rows[:, num_q_heads + num_kv_heads:]


def fused_rope_kv_write(qkv, positions, slot_mapping, k_cache, v_cache, num_q_heads: int, num_kv_heads: int,
                        theta: float):
    """Returns (q_out [T, Hq, D] in qkv's dtype, new k_cache, new v_cache).

    q_out[t] = rope(q[t], positions[t]) rounded to the input type; for every t
    with slot_mapping[t] >= 0, the cache row at (slot // block_size,
    slot % block_size) receives rope(k[t]) rounded to the input type and the
    unchanged bits of v[t].  All other cache bytes are kept as they were."""
    q, k, v = split_qkv(qkv, num_q_heads, num_kv_heads)
    dtype = qkv.dtype
    q_out = rope(q, positions, theta).to(dtype)
    k_rot = rope(k, positions, theta).to(dtype)
    block_size = k_cache.shape[1]
    k_bits = k_cache.view(torch.int16).clone()
    v_bits = v_cache.view(torch.int16).clone()
    k_rot_bits = k_rot.view(torch.int16)
    v_in_bits = v.contiguous().view(torch.int16)
    for t in range(len(slot_mapping)):
        slot = int(slot_mapping[t])
        if slot < 0:
            continue
        block, offset = slot // block_size, slot % block_size
        k_bits[block, offset] = k_rot_bits[t]
        v_bits[block, offset] = v_in_bits[t]
    return q_out, k_bits.view(k_cache.dtype), v_bits.view(v_cache.dtype)

