"""Seeded synthetic paged-attention inputs.

Every function here draws random numbers and lays them out; none of it
computes attention.  Shapes and value distributions follow the workloads the
pages measure:

* MiniLLM Runtime, "CUDA PagedAttention scope" and "Key benchmark results":
  one fp16 request, 2 heads, head dim 64, KV block size 16, contexts of 128,
  1,024 and 4,096 tokens.
* mini_engine, "Custom CUDA kernels" and "Results": bf16 Qwen3-0.6B attention
  shape (16 query heads, 8 KV heads, head dim 128, block 16), prompts and
  outputs of 100-1,024 tokens with a 2,048-token model length, 256 requests,
  and the online mixture of 90% short (128-512) and 10% long (4,096-7,680)
  prompts under a per-step token budget with decodes scheduled first.
* miniserve, "Engine" flowchart: new K/V rows go to
  ``slot = block_id * block_size + offset`` before attention runs.

Layout of the returned KV pool: ``k_cache`` and ``v_cache`` are separate
tensors of shape ``[num_blocks, block_size, num_kv_heads, head_dim]`` (token
major inside a block), so the flattened ``[num_blocks * block_size, ...]`` view
is indexed by the slot number.

Random streams: one ``numpy.random.SeedSequence(seed)`` is split into a
structure stream (lengths, tables, sharing) and a value stream (K, V, q and
the new rows, in that order), both PCG64 generators.  Values are drawn as
float32 N(0, 1) and rounded to fp16/bf16 by torch (round to nearest even).

Poisoning (``poison=True``): every slot that no sequence owns, every slot past
a sequence's context inside its last block, the whole sentinel block used for
block-table padding, and every slot the step's KV write is about to fill are set
to NaN, so any read of a slot that should not be read shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = [
    "PagedStep",
    "make_decode_step",
    "make_prefill_step",
    "make_mixed_step",
    "config_1",
    "config_2",
    "config_3",
    "config_4",
    "config_5",
    "CONFIG_NAMES",
]

_VALUE_CHUNK_ELEMS = 1 << 22  # float32 draw buffer, reused for every chunk


@dataclass
class PagedStep:
    """One layer's paged-attention inputs, as host tensors.

    Rows of ``q`` hold the decode rows first (one per decode sequence), then
    the packed prefill rows.  Sequences follow the same order:
    ``block_tables[:num_decode]`` / ``context_lens[:num_decode]`` describe the
    decode sequences and the rest describe the prefill sequences, whose rows
    are ``q[num_decode + query_start_loc[j] : num_decode + query_start_loc[j+1]]``.

    ``context_lens[s]`` counts every token sequence ``s`` attends to, including
    the current decode token or the whole current chunk (their K/V are written
    by ``slot_mapping`` before attention runs).
    """

    name: str
    seed: int
    dtype: torch.dtype
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    scale: float
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    q: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    num_decode: int
    query_start_loc: torch.Tensor
    new_k: torch.Tensor | None
    new_v: torch.Tensor | None
    slot_mapping: torch.Tensor | None
    sentinel_block: int
    refcount: np.ndarray
    poisoned: bool
    meta: dict = field(default_factory=dict)
    # Position (logical token index) of every new row, in q-row order.
    positions: torch.Tensor | None = None

    # ---- derived sizes -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.numel())

    @property
    def num_prefill(self) -> int:
        return self.num_seqs - self.num_decode

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def num_rows(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_prefill_rows(self) -> int:
        return self.num_rows - self.num_decode

    @property
    def max_query_len(self) -> int:
        if self.num_prefill == 0:
            return 0
        qsl = self.query_start_loc
        return int((qsl[1:] - qsl[:-1]).max())

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.num_seqs else 0

    @property
    def decode_q(self) -> torch.Tensor:
        return self.q[: self.num_decode]

    @property
    def prefill_q(self) -> torch.Tensor:
        return self.q[self.num_decode:]

    @property
    def decode_block_tables(self) -> torch.Tensor:
        return self.block_tables[: self.num_decode]

    @property
    def prefill_block_tables(self) -> torch.Tensor:
        return self.block_tables[self.num_decode:]

    @property
    def decode_context_lens(self) -> torch.Tensor:
        return self.context_lens[: self.num_decode]

    @property
    def prefill_context_lens(self) -> torch.Tensor:
        return self.context_lens[self.num_decode:]


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    structure, values = ss.spawn(2)
    return np.random.default_rng(structure), np.random.default_rng(values)


def _normal(gen: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    """float32 N(0,1) draws rounded to ``dtype`` (nearest even), drawn through
    one reused float32 buffer so big pools need no big temporaries."""
    out = torch.empty(shape, dtype=dtype)
    flat = out.view(-1)
    n = flat.numel()
    buf = np.empty(min(_VALUE_CHUNK_ELEMS, max(n, 1)), dtype=np.float32)
    pos = 0
    while pos < n:
        take = min(buf.size, n - pos)
        gen.standard_normal(out=buf[:take], dtype=np.float32)
        flat[pos: pos + take].copy_(torch.from_numpy(buf[:take]))
        pos += take
    return out


def _assign_blocks(rng, blocks_per_seq, sharing, prefix_blocks, num_blocks):
    """Give each sequence physical block ids from one seeded permutation.

    Sequences with ``sharing[s]`` start with the same ``prefix_blocks`` ids
    (one shared prefix); every other logical block gets a distinct id.
    Returns (tables as lists, ids nobody owns).
    """
    perm = rng.permutation(num_blocks)
    cursor = 0
    prefix_ids: list[int] = []
    if any(sharing):
        prefix_ids = [int(x) for x in perm[:prefix_blocks]]
        cursor = prefix_blocks
    tables = []
    for nb, sh in zip(blocks_per_seq, sharing):
        row = list(prefix_ids) if sh else []
        rest = nb - len(row)
        if rest < 0:
            raise ValueError("a sharing sequence must be longer than the shared prefix")
        row.extend(int(x) for x in perm[cursor: cursor + rest])
        cursor += rest
        tables.append(row)
    if cursor > num_blocks:
        raise ValueError("pool too small")
    unowned = [int(x) for x in perm[cursor:]]
    return tables, unowned


def _build(
    *,
    name: str,
    seed: int,
    dtype: torch.dtype,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    decode_ctx: list[int],
    prefill_cached: list[int],
    prefill_qlen: list[int],
    sharing: list[bool] | None,
    prefix_len: int,
    num_blocks: int | None,
    pool_factor: float,
    write_new: bool,
    poison: bool,
    rng,
    vgen,
    meta: dict | None = None,
) -> PagedStep:
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    B = block_size
    nd = len(decode_ctx)
    ctx = list(decode_ctx) + [c + q for c, q in zip(prefill_cached, prefill_qlen)]
    S = len(ctx)
    if sharing is None:
        sharing = [False] * S
    prefix_blocks = prefix_len // B if any(sharing) else 0
    if any(sharing) and prefix_len % B:
        raise ValueError("shared prefix must be whole blocks")
    blocks_per_seq = [-(-c // B) for c in ctx]
    distinct = sum(nb - (prefix_blocks if sh else 0) for nb, sh in zip(blocks_per_seq, sharing))
    distinct += prefix_blocks
    if num_blocks is None:
        num_blocks = max(int(math.ceil(pool_factor * distinct)), distinct + 1)
    if num_blocks < distinct + 1:
        raise ValueError("pool needs one unowned block for the padding sentinel")
    tables, unowned = _assign_blocks(rng, blocks_per_seq, sharing, prefix_blocks, num_blocks)
    sentinel = unowned[0]
    width = max(blocks_per_seq) if S else 1
    bt = np.full((S, width), sentinel, dtype=np.int32)
    for s, row in enumerate(tables):
        bt[s, : len(row)] = row
    refcount = np.zeros(num_blocks, dtype=np.int64)
    for row in tables:
        for b in row:
            refcount[b] += 1

    # K/V pool, then queries, then the new rows (fixed draw order per seed).
    Hkv, D, Hq = num_kv_heads, head_dim, num_q_heads
    k_cache = _normal(vgen, (num_blocks, B, Hkv, D), dtype)
    v_cache = _normal(vgen, (num_blocks, B, Hkv, D), dtype)
    num_rows = nd + sum(prefill_qlen)
    q = _normal(vgen, (num_rows, Hq, D), dtype)

    # Positions written by this step, per sequence.
    new_positions: list[list[int]] = []
    for s in range(S):
        if s < nd:
            new_positions.append([ctx[s] - 1])
        else:
            j = s - nd
            c = prefill_cached[j]
            new_positions.append(list(range(c, c + prefill_qlen[j])))

    new_k = new_v = slot_mapping = None
    if write_new:
        slots = []
        for s in range(S):
            for pos in new_positions[s]:
                pb = int(bt[s, pos // B])
                if refcount[pb] > 1:
                    raise AssertionError("a new token may not land in a shared block")
                slots.append(pb * B + pos % B)
        slot_mapping = torch.tensor(slots, dtype=torch.int64)
        new_k = _normal(vgen, (len(slots), Hkv, D), dtype)
        new_v = _normal(vgen, (len(slots), Hkv, D), dtype)

    if poison:
        nan = float("nan")
        owned = refcount > 0
        k_cache[torch.from_numpy(~owned)] = nan
        v_cache[torch.from_numpy(~owned)] = nan
        for s in range(S):
            last = blocks_per_seq[s] - 1
            tail = ctx[s] - last * B
            pb = int(bt[s, last])
            k_cache[pb, tail:] = nan
            v_cache[pb, tail:] = nan
        if write_new:
            fk = k_cache.view(num_blocks * B, Hkv, D)
            fv = v_cache.view(num_blocks * B, Hkv, D)
            fk[slot_mapping] = nan
            fv[slot_mapping] = nan

    qsl = [0]
    for ql in prefill_qlen:
        qsl.append(qsl[-1] + ql)
    info = dict(meta or {})
    info.update(
        distinct_blocks=distinct,
        shared_prefix_blocks=prefix_blocks,
        sharing=list(sharing),
        prefill_cached=list(prefill_cached),
        prefill_qlen=list(prefill_qlen),
    )
    return PagedStep(
        name=name,
        seed=seed,
        dtype=dtype,
        num_q_heads=Hq,
        num_kv_heads=Hkv,
        head_dim=D,
        block_size=B,
        scale=1.0 / math.sqrt(D),
        k_cache=k_cache,
        v_cache=v_cache,
        q=q,
        block_tables=torch.from_numpy(bt),
        context_lens=torch.tensor(ctx, dtype=torch.int32),
        num_decode=nd,
        query_start_loc=torch.tensor(qsl, dtype=torch.int32),
        new_k=new_k,
        new_v=new_v,
        slot_mapping=slot_mapping,
        positions=torch.tensor([p for row in new_positions for p in row], dtype=torch.int64),
        sentinel_block=sentinel,
        refcount=refcount,
        poisoned=poison,
        meta=info,
    )


# ---------------------------------------------------------------------------
# generic builders
# ---------------------------------------------------------------------------


def make_decode_step(
    *,
    context_lens,
    dtype=torch.bfloat16,
    num_q_heads=16,
    num_kv_heads=8,
    head_dim=128,
    block_size=16,
    num_blocks=None,
    pool_factor=1.1,
    write_new=False,
    poison=False,
    seed=0,
    name="decode",
) -> PagedStep:
    """Decode-only step: one query row per sequence, contexts as given."""
    rng, vgen = _streams(seed)
    return _build(
        name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        decode_ctx=[int(c) for c in context_lens], prefill_cached=[], prefill_qlen=[],
        sharing=None, prefix_len=0, num_blocks=num_blocks, pool_factor=pool_factor,
        write_new=write_new, poison=poison, rng=rng, vgen=vgen,
    )


def make_prefill_step(
    *,
    query_lens,
    cached_lens,
    dtype=torch.bfloat16,
    num_q_heads=16,
    num_kv_heads=8,
    head_dim=128,
    block_size=16,
    sharing=None,
    prefix_len=256,
    num_blocks=None,
    pool_factor=1.1,
    write_new=True,
    poison=False,
    seed=0,
    name="prefill",
) -> PagedStep:
    """Prefill-only step: ragged chunks, chunk j has ``query_lens[j]`` rows and
    attends to ``cached_lens[j]`` earlier tokens plus itself (bottom-right)."""
    rng, vgen = _streams(seed)
    return _build(
        name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        decode_ctx=[], prefill_cached=[int(c) for c in cached_lens],
        prefill_qlen=[int(q) for q in query_lens], sharing=sharing, prefix_len=prefix_len,
        num_blocks=num_blocks, pool_factor=pool_factor, write_new=write_new,
        poison=poison, rng=rng, vgen=vgen,
    )


def make_mixed_step(
    *,
    decode_ctx,
    query_lens,
    cached_lens,
    dtype=torch.bfloat16,
    num_q_heads=16,
    num_kv_heads=8,
    head_dim=128,
    block_size=16,
    sharing=None,
    prefix_len=256,
    num_blocks=None,
    pool_factor=1.1,
    write_new=True,
    poison=False,
    seed=0,
    name="mixed",
) -> PagedStep:
    """Decode sequences followed by prefill chunks, sharing one pool and one q."""
    rng, vgen = _streams(seed)
    return _build(
        name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        decode_ctx=[int(c) for c in decode_ctx], prefill_cached=[int(c) for c in cached_lens],
        prefill_qlen=[int(q) for q in query_lens], sharing=sharing, prefix_len=prefix_len,
        num_blocks=num_blocks, pool_factor=pool_factor, write_new=write_new,
        poison=poison, rng=rng, vgen=vgen,
    )


# ---------------------------------------------------------------------------
# the five measured workloads
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "single-request fp16 decode, 2 heads, head_dim 64, ctx 128",
    2: "single-request fp16 decode context sweep (128 / 1024 / 4096)",
    3: "batched GQA bf16 decode, 256 seqs, 16q/8kv, head_dim 128, ctx U[100,2048] + KV write",
    4: "split-K bf16 decode, 4 seqs x 16384 ctx, 16q/8kv, head_dim 128",
    5: "mixed bf16 step: 64 decodes + ragged causal prefill chunks, budget 2048",
}


def config_1(seed=0, poison=False) -> PagedStep:
    """fp16, 2 query heads = 2 KV heads, head dim 64, block 16, one request of
    128 tokens (8 logical blocks) in a 64-block pool."""
    rng, vgen = _streams(seed)
    return _build(
        name="config1", seed=seed, dtype=torch.float16, num_q_heads=2, num_kv_heads=2,
        head_dim=64, block_size=16, decode_ctx=[128], prefill_cached=[], prefill_qlen=[],
        sharing=None, prefix_len=0, num_blocks=64, pool_factor=1.0, write_new=False,
        poison=poison, rng=rng, vgen=vgen,
    )


def config_2(context_len=4096, seed=0, poison=False) -> PagedStep:
    """The config-1 shape at 128, 1,024 or 4,096 tokens, in a pool twice the
    needed size with a seeded random table permutation."""
    if context_len % 16:
        raise ValueError("context sweep lengths are whole blocks")
    rng, vgen = _streams(seed)
    need = context_len // 16
    return _build(
        name=f"config2_ctx{context_len}", seed=seed, dtype=torch.float16, num_q_heads=2,
        num_kv_heads=2, head_dim=64, block_size=16, decode_ctx=[context_len],
        prefill_cached=[], prefill_qlen=[], sharing=None, prefix_len=0,
        num_blocks=2 * need, pool_factor=2.0, write_new=False, poison=poison, rng=rng, vgen=vgen,
    )


def config_3(seed=0, poison=False, num_seqs=256) -> PagedStep:
    """bf16 Qwen3-0.6B attention shape: 256 sequences with context uniform in
    [100, 2048], pool = total blocks + 10 % shuffled; plus one new K/V row per
    sequence at its last position, written before attention."""
    rng, vgen = _streams(seed)
    ctx = [int(x) for x in rng.integers(100, 2049, size=num_seqs)]
    return _build(
        name="config3", seed=seed, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
        head_dim=128, block_size=16, decode_ctx=ctx, prefill_cached=[], prefill_qlen=[],
        sharing=None, prefix_len=0, num_blocks=None, pool_factor=1.1, write_new=True,
        poison=poison, rng=rng, vgen=vgen,
    )


def config_4(seed=0, poison=False) -> PagedStep:
    """bf16, 4 sequences of 16,384 tokens (1,024 blocks each) over a pool of
    4,200 blocks with seeded random tables; long enough for split-K."""
    rng, vgen = _streams(seed)
    return _build(
        name="config4", seed=seed, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
        head_dim=128, block_size=16, decode_ctx=[16384] * 4, prefill_cached=[],
        prefill_qlen=[], sharing=None, prefix_len=0, num_blocks=4200, pool_factor=1.0,
        write_new=False, poison=poison, rng=rng, vgen=vgen,
    )


def config_5(seed=0, poison=False, budget=2048, num_decode=64, max_chunk=512,
             share_frac=0.3, prefix_len=256) -> PagedStep:
    """One mixed scheduler step under a 2,048-token budget.

    * 64 decode sequences, context uniform in [128, 2048], scheduled first.
    * Prefill requests fill the rest of the budget.  Prompt length P is drawn
      90 % uniform in [128, 512] and 10 % uniform in [4096, 7680]; the chunk is
      min(P - c, 512, budget left).  The first prefill request is a long prompt
      part-way through (c = 512 k, k >= 1), so a chunk always attends to earlier
      cached chunks; other requests start at c = 0.
    * Each request longer than the 256-token prefix shares it with probability
      0.3; its table then starts with the same 16 physical blocks, and a sharing
      prefill request has its prefix cached (c >= 256).
    * Pool = 1.1 x distinct blocks, shuffled.
    """
    rng, vgen = _streams(seed)
    decode_ctx = [int(x) for x in rng.integers(128, 2049, size=num_decode)]
    sharing = [bool(c > prefix_len and rng.random() < share_frac) for c in decode_ctx]
    left = budget - num_decode
    cached, qlens, prompt = [], [], []
    first = True
    while left > 0:
        if first:
            P = int(rng.integers(4096, 7681))
            k = int(rng.integers(1, (P - 1) // max_chunk + 1))
            c = max_chunk * k
            first = False
        else:
            if rng.random() < 0.9:
                P = int(rng.integers(128, 513))
            else:
                P = int(rng.integers(4096, 7681))
            c = 0
        share = bool(P > prefix_len and rng.random() < share_frac)
        if share:
            c = max(c, prefix_len)
        chunk = min(P - c, max_chunk, left)
        cached.append(c)
        qlens.append(chunk)
        prompt.append(P)
        sharing.append(share)
        left -= chunk
    return _build(
        name="config5", seed=seed, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
        head_dim=128, block_size=16, decode_ctx=decode_ctx, prefill_cached=cached,
        prefill_qlen=qlens, sharing=sharing, prefix_len=prefix_len, num_blocks=None,
        pool_factor=1.1, write_new=True, poison=poison, rng=rng, vgen=vgen,
        meta=dict(prompt_lens=prompt, budget=budget),
    )


def fused_qkv(step: PagedStep) -> torch.Tensor:
    """The step's new rows as the fused projection output the rotary write
    consumes: [T, (Hq + 2 Hkv) * D] = [q heads | k heads | v heads] per row
    (q from step.q, k and v from step.new_k / step.new_v)."""
    if step.new_k is None:
        raise ValueError("step has no new K/V rows (built with write_new=False)")
    T = step.q.shape[0]
    return torch.cat([step.q, step.new_k, step.new_v], dim=1).reshape(T, -1).contiguous()
