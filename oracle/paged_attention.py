"""CPU fp64 oracle for paged attention over a block-tabled KV cache.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import or call this module.  The GPU library never
calls it and shares no code, header, table or helper with it.

What it computes, and where the pages define it:

* Address translation (MiniLLM Runtime, "Core class relationships"): logical
  token t of a request lies in logical block t // block_size at offset
  t % block_size; the request's block table maps the logical block to a
  physical block of the paged pool.  miniserve's "Engine" flowchart gives the
  flat form slot = block_id * block_size + offset.
* Decode attention (MiniLLM Runtime, "CUDA PagedAttention scope"; mini_engine,
  "Custom CUDA kernels"): one query token per request; QK^T over the whole
  paged context, softmax, weighted sum of V.  Query heads are grouped over KV
  heads (grouped-query attention): the G = Hq / Hkv query heads of a group
  read the same K/V head.
* Split-K decode (mini_engine, "Custom CUDA kernels", paged decode v2): the
  context is cut into fixed-size partitions; each keeps its own max logit and
  exp-sum, and a reduce merges them.
* Prefill (mini_engine, "Custom CUDA kernels", paged prefill attention;
  miniserve, "Engine" flowchart, bottom-right causal mask): a chunk of q rows
  placed at the end of the sequence; row i sees the c = ctx - q cached tokens
  and the chunk's rows up to and including itself.
* KV-cache write (mini_engine, "Custom CUDA kernels", KV-cache write;
  miniserve, "Engine" flowchart, index_copy_ into the paged pool): new rows
  are copied to their slots; padded slots (negative) are skipped.

Method: the plain definition, exactly as written above.  Each request's K and
V are first materialised from the block table (the slow path the pages
replace) and attention is the textbook two-pass softmax in float64.  The
softmax scale is an explicit argument applied to the dot products.  fp16 and
bf16 inputs are widened to float64 exactly before any arithmetic.

Readings where the pages are silent (listed again in the design notes):
the KV pool is ``[num_blocks, block_size, num_kv_heads, head_dim]`` per tensor;
query head h uses KV head h // G; context_lens include the current token or
the whole current chunk; negative slots are padding; the exponential is the
natural one.
"""

from __future__ import annotations

import torch

__all__ = [
    "widen",
    "kv_head_of",
    "token_location",
    "materialize",
    "attend",
    "visible_keys",
    "decode",
    "prefill",
    "decode_partitions",
    "merge_partitions",
    "kv_cache_write",
]

F64 = torch.float64


def widen(x: torch.Tensor) -> torch.Tensor:
    """fp16 / bf16 / fp32 -> float64.  Exact: every fp16, bf16 and fp32 value
    is representable in float64."""
    return x.to(F64)


def kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """KV head read by query head ``h``: consecutive query heads form a group
    of G = num_q_heads // num_kv_heads that share one KV head."""
    group = num_q_heads // num_kv_heads
    return h // group


def token_location(t: torch.Tensor, table_row: torch.Tensor, block_size: int):
    """Logical token index -> (physical block, offset in the block)."""
    logical_block = t // block_size
    offset = t % block_size
    return table_row[logical_block].to(torch.int64), offset


def materialize(cache: torch.Tensor, table_row: torch.Tensor, ctx: int) -> torch.Tensor:
    """Gather one request's first ``ctx`` tokens of ``cache`` through its block
    table into a contiguous float64 tensor ``[ctx, num_kv_heads, head_dim]``."""
    block_size = cache.shape[1]
    t = torch.arange(ctx, dtype=torch.int64)
    pb, off = token_location(t, table_row, block_size)
    return widen(cache[pb, off])


def attend(q_vec: torch.Tensor, keys: torch.Tensor, values: torch.Tensor, scale: float) -> torch.Tensor:
    """Textbook softmax attention of one query over n keys (all float64):
    s_t = scale * <q, k_t>;  m = max_t s_t;  w_t = exp(s_t - m);
    out = sum_t w_t v_t / sum_t w_t."""
    s = scale * (keys @ q_vec)
    m = s.max()
    w = torch.exp(s - m)
    return (w @ values) / w.sum()


def visible_keys(cached: int, row: int) -> int:
    """Number of keys row ``row`` of a chunk sees when ``cached`` tokens
    precede the chunk: every cached token and the chunk rows 0..row
    (the bottom-right causal mask)."""
    return cached + row + 1


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, seqs=None) -> torch.Tensor:
    """Paged decode: ``q [S, Hq, D]`` (one token per sequence) -> float64
    ``out [S, Hq, D]`` (or only the rows listed in ``seqs``, in that order)."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    rows = range(S) if seqs is None else [int(s) for s in seqs]
    out = torch.empty((len(rows), Hq, D), dtype=F64)
    for r, s in enumerate(rows):
        ctx = int(context_lens[s])
        K = materialize(k_cache, block_tables[s], ctx)
        V = materialize(v_cache, block_tables[s], ctx)
        qs = widen(q[s])
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            out[r, h] = attend(qs[h], K[:, g], V[:, g], scale)
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start_loc, scale, seqs=None,
            rows=None) -> torch.Tensor:
    """Paged prefill over ragged chunks.  ``q [Nq, Hq, D]`` holds the chunks
    packed back to back; chunk j is rows ``query_start_loc[j]`` to
    ``query_start_loc[j+1]`` and its sequence has ``context_lens[j]`` tokens in
    the cache, the chunk's own rows being the last ones.  Returns float64
    ``[Nq, Hq, D]``; only chunks listed in ``seqs`` and packed rows listed in
    ``rows`` are computed (default: all), the others are left NaN."""
    Nq, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    out = torch.full((Nq, Hq, D), float("nan"), dtype=F64)
    nseq = len(query_start_loc) - 1
    chunks = range(nseq) if seqs is None else [int(s) for s in seqs]
    wanted = None if rows is None else {int(r) for r in rows}
    for j in chunks:
        start, end = int(query_start_loc[j]), int(query_start_loc[j + 1])
        qlen = end - start
        if qlen == 0:
            continue
        if wanted is not None and not any(start <= r < end for r in wanted):
            continue
        ctx = int(context_lens[j])
        cached = ctx - qlen
        if cached < 0:
            raise ValueError("a chunk cannot be longer than its context")
        K = materialize(k_cache, block_tables[j], ctx)
        V = materialize(v_cache, block_tables[j], ctx)
        for i in range(qlen):
            if wanted is not None and start + i not in wanted:
                continue
            n = visible_keys(cached, i)
            qi = widen(q[start + i])
            for h in range(Hq):
                g = kv_head_of(h, Hq, Hkv)
                out[start + i, h] = attend(qi[h], K[:n, g], V[:n, g], scale)
    return out


def decode_partitions(q, k_cache, v_cache, block_tables, context_lens, scale, partition_size, seqs=None):
    """Per-partition decode state.  Partition p of sequence s covers logical
    tokens [p * P, min((p + 1) * P, ctx)).  For each (s, h, p) it returns the
    max logit m_p, the exp-sum l_p = sum exp(s_t - m_p) and the normalised
    partial output o_p = sum exp(s_t - m_p) v_t / l_p.  Partitions past the end
    of a sequence are marked by num_partitions[s].

    Returns (max_logits [S, Hq, Pmax], exp_sums [S, Hq, Pmax],
    partial_out [S, Hq, Pmax, D], num_partitions [S]) in float64; unused
    partition slots hold NaN."""
    S, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    rows = range(S) if seqs is None else [int(s) for s in seqs]
    ctxs = [int(context_lens[s]) for s in rows]
    pmax = max(-(-c // partition_size) for c in ctxs) if ctxs else 0
    n = len(ctxs)
    max_logits = torch.full((n, Hq, pmax), float("nan"), dtype=F64)
    exp_sums = torch.full((n, Hq, pmax), float("nan"), dtype=F64)
    partial = torch.full((n, Hq, pmax, D), float("nan"), dtype=F64)
    nparts = torch.zeros(n, dtype=torch.int64)
    for r, s in enumerate(rows):
        ctx = ctxs[r]
        K = materialize(k_cache, block_tables[s], ctx)
        V = materialize(v_cache, block_tables[s], ctx)
        qs = widen(q[s])
        P = -(-ctx // partition_size)
        nparts[r] = P
        for h in range(Hq):
            g = kv_head_of(h, Hq, Hkv)
            for p in range(P):
                lo, hi = p * partition_size, min((p + 1) * partition_size, ctx)
                sc = scale * (K[lo:hi, g] @ qs[h])
                m = sc.max()
                w = torch.exp(sc - m)
                max_logits[r, h, p] = m
                exp_sums[r, h, p] = w.sum()
                partial[r, h, p] = (w @ V[lo:hi, g]) / w.sum()
    return max_logits, exp_sums, partial, nparts


def merge_partitions(max_logits, exp_sums, partial_out, num_partitions) -> torch.Tensor:
    """Merge per-partition states: M = max_p m_p, w_p = l_p exp(m_p - M),
    out = sum_p w_p o_p / sum_p w_p over the sequence's valid partitions."""
    n, Hq, _ = max_logits.shape
    D = partial_out.shape[-1]
    out = torch.empty((n, Hq, D), dtype=F64)
    for r in range(n):
        P = int(num_partitions[r])
        for h in range(Hq):
            m = max_logits[r, h, :P]
            M = m.max()
            w = exp_sums[r, h, :P] * torch.exp(m - M)
            out[r, h] = (w @ partial_out[r, h, :P]) / w.sum()
    return out


def kv_cache_write(key, value, slot_mapping, k_cache, v_cache):
    """Scatter new K/V rows into the paged pool: row i goes to physical block
    slot // block_size at offset slot % block_size; rows whose slot is
    negative are padding and are skipped.  Works on the raw 16-bit patterns, so
    the copy is bit-exact and every untouched byte (NaN payloads included) is
    kept.  Returns new (k_cache, v_cache); the inputs are not modified."""
    block_size = k_cache.shape[1]
    k_bits = k_cache.view(torch.int16).clone()
    v_bits = v_cache.view(torch.int16).clone()
    key_bits = key.view(torch.int16)
    value_bits = value.view(torch.int16)
    for i in range(len(slot_mapping)):
        slot = int(slot_mapping[i])
        if slot < 0:
            continue
        block, offset = slot // block_size, slot % block_size
        k_bits[block, offset] = key_bits[i]
        v_bits[block, offset] = value_bits[i]
    return k_bits.view(k_cache.dtype), v_bits.view(v_cache.dtype)
