"""Pins for the CPU oracle: checks that fix what it computes without trusting
it.  Each ``check_*`` takes the oracle module and raises AssertionError when
the oracle disagrees with what the definitions or the mathematics fix:

* hand-derived worked examples (tests/golden/*.json, each citing the
  definition it follows);
* closed forms: a one-token context returns V exactly; constant keys or a
  zero scale give the plain mean of V; one overwhelming key returns its V;
* invariants: relabelling physical blocks changes nothing (bit for bit);
  (alpha q, scale / alpha) changes nothing; GQA equals MHA with each KV head
  repeated for its query heads; split-K merged over any partition size equals
  the unsplit result; chunking a prompt changes no row; keys after a row's
  position do not affect it;
* library special cases: on a contiguous pool the result equals
  torch.nn.functional.scaled_dot_product_attention in float64, with an
  explicit bottom-right boolean mask for prefill;
* brute force over tiny pools against a second formulation written
  differently: pure-Python per-token slot reads and a log-sum-exp softmax.

The module holds no test functions itself (tests/test_oracle_pins.py calls
every check; tests/test_oracle_mutants.py plants mistakes in the oracle and
expects some check to fail).
"""

from __future__ import annotations

import itertools
import json
import math
import os

import torch
import torch.nn.functional as F

from workloads import make_decode_step, make_prefill_step

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F64 = torch.float64


# ---------------------------------------------------------------------------
# small independent helpers (not shared with the oracle)
# ---------------------------------------------------------------------------


def _rows_by_slot(cache, table_row, ctx):
    """Gather through the flat slot formula slot = block * block_size + offset."""
    B = cache.shape[1]
    flat = cache.reshape(cache.shape[0] * B, *cache.shape[2:])
    slots = [int(table_row[t // B]) * B + t % B for t in range(ctx)]
    return flat[slots].to(F64)


def _lse_decode_row(qv, flat_k, flat_v, table_row, ctx, B, g, scale):
    """Second formulation in pure Python: per-token slot reads, logits,
    log-sum-exp, then exp(logit - lse)-weighted values."""
    D = len(qv)
    logits = []
    vals = []
    for t in range(ctx):
        slot = int(table_row[t // B]) * B + t % B
        k = flat_k[slot][g]
        logits.append(scale * math.fsum(qv[d] * k[d] for d in range(D)))
        vals.append(flat_v[slot][g])
    mx = max(logits)
    lse = mx + math.log(math.fsum(math.exp(x - mx) for x in logits))
    return [math.fsum(math.exp(logits[t] - lse) * vals[t][d] for t in range(ctx)) for d in range(D)]


def _sdpa(q, k, v, scale, mask=None):
    """torch SDPA in float64 on CPU.  q [Hq, n, D], k/v [Hq, m, D]."""
    return F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)


def _assert_close(a, b, tol, what):
    a = torch.as_tensor(a, dtype=F64)
    b = torch.as_tensor(b, dtype=F64)
    assert a.shape == b.shape, f"{what}: shape {tuple(a.shape)} vs {tuple(b.shape)}"
    assert torch.isfinite(a).all(), f"{what}: non-finite values"
    err = (a - b).abs().max().item() if a.numel() else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _dec(o, step, **kw):
    return o.decode(step.decode_q, step.k_cache, step.v_cache, step.decode_block_tables,
                    step.decode_context_lens, kw.pop("scale", step.scale), **kw)


def _pre(o, step, **kw):
    return o.prefill(step.prefill_q, step.k_cache, step.v_cache, step.prefill_block_tables,
                     step.prefill_context_lens, step.query_start_loc, kw.pop("scale", step.scale), **kw)


def _small_decode(ctx, seed, Hq=4, Hkv=2, D=8, dtype=torch.float16, poison=True):
    return make_decode_step(context_lens=ctx, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
                            head_dim=D, seed=seed, poison=poison, pool_factor=1.5)


def _load_golden():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)

    def num(x):
        if isinstance(x, list) and x and x[0] == "ln":
            return math.log(x[1])
        if isinstance(x, list) and x and x[0] == "frac":
            return x[1] / x[2]
        return float(x)

    B, NB = g["block_size"], g["num_blocks"]
    D = 2
    k = torch.full((NB, B, 1, D), float("nan"), dtype=F64)
    v = torch.full((NB, B, 1, D), float("nan"), dtype=F64)
    table = g["block_table"]
    for t, (kr, vr) in enumerate(zip(g["k_rows_by_logical_token"], g["v_rows_by_logical_token"])):
        pb, off = table[t // B], t % B
        k[pb, off, 0] = torch.tensor([num(x) for x in kr], dtype=F64)
        v[pb, off, 0] = torch.tensor([num(x) for x in vr], dtype=F64)
    conv = lambda rows: torch.tensor([[[num(x) for x in r] for r in h] for h in rows], dtype=F64)  # noqa: E731
    return dict(
        k=k, v=v, table=torch.tensor([table], dtype=torch.int32),
        ctx=torch.tensor([g["context_len"]], dtype=torch.int32), scale=g["scale"],
        q_decode=torch.tensor([g["q_decode"]], dtype=F64),
        decode_out=torch.tensor([[[num(x) for x in r] for r in g["decode_out"]]], dtype=F64),
        q_prefill=torch.tensor(g["q_prefill"], dtype=F64),
        qsl=torch.tensor(g["query_start_loc"], dtype=torch.int32),
        prefill_out=conv(g["prefill_out"]),
    )


# ---------------------------------------------------------------------------
# decode pins
# ---------------------------------------------------------------------------


def check_golden_decode(o):
    g = _load_golden()
    out = o.decode(g["q_decode"], g["k"], g["v"], g["table"], g["ctx"], g["scale"])
    _assert_close(out, g["decode_out"], 1e-12, "hand-derived decode example")


def check_context_of_one_returns_v(o):
    step = _small_decode([1, 1, 1], seed=11)
    out = _dec(o, step)
    for s in range(step.num_decode):
        v0 = _rows_by_slot(step.v_cache, step.block_tables[s], 1)[0]
        for h in range(step.num_q_heads):
            g = h // (step.num_q_heads // step.num_kv_heads)
            assert torch.equal(out[s, h], v0[g]), "ctx 1 must return V exactly"


def check_constant_keys_give_mean_of_v(o):
    step = _small_decode([5, 16, 17, 40], seed=12)
    kc = step.k_cache.clone()
    kc[:] = torch.randn(step.num_kv_heads, step.head_dim, generator=torch.Generator().manual_seed(3)).to(kc.dtype)
    out = o.decode(step.decode_q, kc, step.v_cache, step.decode_block_tables, step.decode_context_lens, step.scale)
    G = step.num_q_heads // step.num_kv_heads
    for s in range(step.num_decode):
        V = _rows_by_slot(step.v_cache, step.block_tables[s], int(step.context_lens[s]))
        for h in range(step.num_q_heads):
            _assert_close(out[s, h], V[:, h // G].mean(0), 1e-13, "constant keys -> mean of V")


def check_zero_scale_gives_mean_of_v(o):
    step = _small_decode([3, 33, 64], seed=13)
    out = _dec(o, step, scale=0.0)
    G = step.num_q_heads // step.num_kv_heads
    for s in range(step.num_decode):
        V = _rows_by_slot(step.v_cache, step.block_tables[s], int(step.context_lens[s]))
        for h in range(step.num_q_heads):
            _assert_close(out[s, h], V[:, h // G].mean(0), 1e-13, "scale 0 -> mean of V")


def check_dominant_key_selects_its_value(o):
    step = _small_decode([37], seed=14, Hq=2, Hkv=2, D=8, dtype=torch.float32)
    K = _rows_by_slot(step.k_cache, step.block_tables[0], 37)
    V = _rows_by_slot(step.v_cache, step.block_tables[0], 37)
    j = 23
    q = torch.zeros(1, 2, 8, dtype=torch.float32)
    kc = step.k_cache.clone()
    # make every key orthogonal-ish small except key j, which aligns with q
    B = step.block_size
    for t in range(37):
        pb, off = int(step.block_tables[0][t // B]), t % B
        kc[pb, off] = 0.0
    pb, off = int(step.block_tables[0][j // B]), j % B
    kc[pb, off] = K[j].to(torch.float32)
    for h in range(2):
        q[0, h] = K[j, h].to(torch.float32)
    out = o.decode(q, kc, step.v_cache, step.decode_block_tables, step.decode_context_lens, 1000.0)
    for h in range(2):
        _assert_close(out[0, h], V[j, h], 1e-12, "overwhelming key -> its value")


def check_block_permutation_invariance(o):
    step = _small_decode([7, 16, 31, 48, 49], seed=15)
    base = _dec(o, step)
    NB = step.num_blocks
    perm = torch.randperm(NB, generator=torch.Generator().manual_seed(5))  # new id of old block b
    kc = torch.empty_like(step.k_cache)
    vc = torch.empty_like(step.v_cache)
    kc[perm] = step.k_cache
    vc[perm] = step.v_cache
    bt = perm[step.block_tables.long()].to(torch.int32)
    out = o.decode(step.decode_q, kc, vc, bt, step.decode_context_lens, step.scale)
    assert torch.equal(out, base), "relabelling physical blocks must not change a bit"


def check_brute_force_tiny_pools(o):
    """Every injective table of 3 logical blocks over a 5-block pool, contexts
    1..48 (block 16), against the pure-Python log-sum-exp formulation."""
    B, D, Hq, Hkv, NB = 16, 4, 2, 1, 5
    gen = torch.Generator().manual_seed(21)
    kc = torch.randn(NB, B, Hkv, D, generator=gen, dtype=F64)
    vc = torch.randn(NB, B, Hkv, D, generator=gen, dtype=F64)
    q = torch.randn(1, Hq, D, generator=gen, dtype=F64)
    flat_k = kc.reshape(NB * B, Hkv, D).tolist()
    flat_v = vc.reshape(NB * B, Hkv, D).tolist()
    tables = list(itertools.permutations(range(NB), 3))
    ctxs = [1, 2, 15, 16, 17, 31, 32, 33, 47, 48]
    for n_t, table in enumerate(tables):
        bt = torch.tensor([table], dtype=torch.int32)
        for ctx in ctxs[n_t % 2::2]:
            out = o.decode(q, kc, vc, bt, torch.tensor([ctx], dtype=torch.int32), 0.7)
            for h in range(Hq):
                ref = _lse_decode_row(q[0, h].tolist(), flat_k, flat_v, table, ctx, B, h // (Hq // Hkv), 0.7)
                _assert_close(out[0, h], ref, 1e-12, f"brute force table {table} ctx {ctx}")


def check_contiguous_pool_matches_sdpa(o):
    """Identity block table over a contiguous pool: plain SDPA (library)."""
    B, NB, Hkv, D = 16, 6, 3, 16
    gen = torch.Generator().manual_seed(22)
    kc = torch.randn(NB, B, Hkv, D, generator=gen, dtype=F64)
    vc = torch.randn(NB, B, Hkv, D, generator=gen, dtype=F64)
    q = torch.randn(1, Hkv, D, generator=gen, dtype=F64)
    for ctx in (1, 9, 16, 50, 96):
        bt = torch.arange(NB, dtype=torch.int32)[None]
        out = o.decode(q, kc, vc, bt, torch.tensor([ctx], dtype=torch.int32), 0.25)
        K = kc.reshape(NB * B, Hkv, D)[:ctx].transpose(0, 1)
        V = vc.reshape(NB * B, Hkv, D)[:ctx].transpose(0, 1)
        ref = _sdpa(q[0][:, None, :], K, V, 0.25)[:, 0, :]
        _assert_close(out[0], ref, 1e-12, f"SDPA on contiguous pool ctx {ctx}")


def check_gqa_equals_mha_with_repeated_kv(o):
    step = _small_decode([9, 30, 64], seed=16, Hq=6, Hkv=2)
    G = step.num_q_heads // step.num_kv_heads
    out = _dec(o, step)
    rep = lambda c: c.repeat_interleave(G, dim=2)  # noqa: E731  kv head g -> q heads gG..gG+G-1
    mha = o.decode(step.decode_q, rep(step.k_cache), rep(step.v_cache), step.decode_block_tables,
                   step.decode_context_lens, step.scale)
    _assert_close(out, mha, 1e-14, "GQA vs MHA with repeated KV heads")


def check_scale_invariance(o):
    step = _small_decode([20, 45], seed=17, dtype=torch.float32)
    out = _dec(o, step)
    q3 = step.decode_q.to(F64) * 3.0
    out3 = o.decode(q3, step.k_cache, step.v_cache, step.decode_block_tables, step.decode_context_lens,
                    step.scale / 3.0)
    _assert_close(out3, out, 1e-12, "(3 q, scale / 3)")


def check_never_reads_unowned_slots(o):
    """Poisoned pool (NaN in every unowned slot, block tail and table padding)."""
    step = _small_decode([1, 15, 16, 17, 33], seed=18)
    assert torch.isnan(step.k_cache).any()
    out = _dec(o, step)
    assert torch.isfinite(out).all(), "an unowned slot was read"


# ---------------------------------------------------------------------------
# split-K pins
# ---------------------------------------------------------------------------


def check_splitk_merge_equals_unsplit(o):
    step = _small_decode([1, 16, 255, 256, 257, 600], seed=19, Hq=2, Hkv=1, D=8)
    ref = _dec(o, step)
    for P in (1, 16, 256, 600):
        m, l, po, npart = o.decode_partitions(step.decode_q, step.k_cache, step.v_cache,
                                              step.decode_block_tables, step.decode_context_lens,
                                              step.scale, P)
        out = o.merge_partitions(m, l, po, npart)
        rel = ((out - ref).abs().max() / ref.abs().max()).item()
        assert rel <= 1e-12, f"split-K merge with partition {P}: rel err {rel:.2e}"


def check_splitk_partition_state(o):
    """A one-token partition has l = 1, o = v and m = its logit; the partition
    count is ceil(ctx / P)."""
    step = _small_decode([3, 5], seed=20, Hq=2, Hkv=2, D=8)
    m, l, po, npart = o.decode_partitions(step.decode_q, step.k_cache, step.v_cache,
                                          step.decode_block_tables, step.decode_context_lens, step.scale, 1)
    assert npart.tolist() == [3, 5]
    for s in range(2):
        ctx = int(step.context_lens[s])
        K = _rows_by_slot(step.k_cache, step.block_tables[s], ctx)
        V = _rows_by_slot(step.v_cache, step.block_tables[s], ctx)
        qs = step.decode_q[s].to(F64)
        for h in range(2):
            for t in range(ctx):
                assert l[s, h, t].item() == 1.0
                assert torch.equal(po[s, h, t], V[t, h])
                _assert_close(m[s, h, t], step.scale * float((qs[h] * K[t, h]).sum()), 1e-14, "partition logit")
    m4, l4, po4, n4 = o.decode_partitions(step.decode_q, step.k_cache, step.v_cache,
                                          step.decode_block_tables, step.decode_context_lens, step.scale, 4)
    assert n4.tolist() == [1, 2]


# ---------------------------------------------------------------------------
# prefill pins
# ---------------------------------------------------------------------------


def check_golden_prefill(o):
    g = _load_golden()
    out = o.prefill(g["q_prefill"], g["k"], g["v"], g["table"], g["ctx"], g["qsl"], g["scale"])
    _assert_close(out, g["prefill_out"], 1e-12, "hand-derived prefill example")


def check_prefill_matches_sdpa_bottom_right(o):
    """Identity tables: row i of a chunk after c cached tokens attends to keys
    j <= c + i.  Library: SDPA with an explicit boolean mask; for c = 0 also
    SDPA with is_causal=True."""
    B, Hkv, Hq, D = 16, 2, 4, 8
    gen = torch.Generator().manual_seed(23)
    for cached, qlen in ((0, 1), (0, 37), (5, 11), (32, 16), (40, 33)):
        ctx = cached + qlen
        NB = -(-ctx // B)
        kc = torch.randn(NB, B, Hkv, D, generator=gen, dtype=F64)
        vc = torch.randn(NB, B, Hkv, D, generator=gen, dtype=F64)
        q = torch.randn(qlen, Hq, D, generator=gen, dtype=F64)
        bt = torch.arange(NB, dtype=torch.int32)[None]
        out = o.prefill(q, kc, vc, bt, torch.tensor([ctx], dtype=torch.int32),
                        torch.tensor([0, qlen], dtype=torch.int32), 0.3)
        K = kc.reshape(NB * B, Hkv, D)[:ctx].repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
        V = vc.reshape(NB * B, Hkv, D)[:ctx].repeat_interleave(Hq // Hkv, dim=1).transpose(0, 1)
        mask = torch.arange(ctx)[None, :] <= (cached + torch.arange(qlen))[:, None]
        ref = _sdpa(q.transpose(0, 1), K, V, 0.3, mask).transpose(0, 1)
        _assert_close(out, ref, 1e-12, f"prefill vs SDPA mask c={cached} q={qlen}")
        if cached == 0:
            ref2 = F.scaled_dot_product_attention(q.transpose(0, 1), K, V, is_causal=True, scale=0.3).transpose(0, 1)
            _assert_close(out, ref2, 1e-12, f"prefill vs SDPA is_causal q={qlen}")


def check_prefill_chunk_invariance(o):
    """One prompt as a single chunk, or as chunks each attending to the
    earlier cached ones: identical rows, bit for bit."""
    L, chunk = 70, 32
    step = make_prefill_step(query_lens=[L], cached_lens=[0], dtype=torch.float16, num_q_heads=4,
                             num_kv_heads=2, head_dim=8, seed=24, write_new=False)
    whole = _pre(o, step)
    starts = list(range(0, L, chunk))
    qsl = [0]
    ctxs = []
    for s0 in starts:
        n = min(chunk, L - s0)
        qsl.append(qsl[-1] + n)
        ctxs.append(s0 + n)
    bt = step.block_tables.repeat(len(starts), 1)
    out = o.prefill(step.q, step.k_cache, step.v_cache, bt, torch.tensor(ctxs, dtype=torch.int32),
                    torch.tensor(qsl, dtype=torch.int32), step.scale)
    assert torch.equal(out, whole), "chunking a prompt must not change any row"


def check_prefill_rows_equal_decode(o):
    """A one-row chunk equals decode at the same context, and the last row of
    any chunk equals decode at that chunk's context (bit for bit)."""
    step = make_prefill_step(query_lens=[1, 9, 20], cached_lens=[30, 0, 17], dtype=torch.bfloat16,
                             num_q_heads=4, num_kv_heads=2, head_dim=8, seed=25, write_new=False,
                             poison=True)
    out = _pre(o, step)
    qsl = step.query_start_loc.tolist()
    last_rows = [qsl[j + 1] - 1 for j in range(step.num_prefill)]
    dec = o.decode(step.q[last_rows], step.k_cache, step.v_cache, step.block_tables,
                   step.context_lens, step.scale)
    assert torch.equal(out[last_rows], dec), "last chunk row must equal decode"


def check_prefill_causality(o):
    """Changing K/V at positions after row i's leaves row i unchanged and
    changes some later row."""
    step = make_prefill_step(query_lens=[24], cached_lens=[10], dtype=torch.float32, num_q_heads=2,
                             num_kv_heads=1, head_dim=8, seed=26, write_new=False)
    base = _pre(o, step)
    pos = 10 + 13  # chunk row 13's own position; perturb everything after it
    kc, vc = step.k_cache.clone(), step.v_cache.clone()
    B = step.block_size
    for t in range(pos + 1, 34):
        pb, off = int(step.block_tables[0][t // B]), t % B
        kc[pb, off] += 1.0
        vc[pb, off] -= 2.0
    out = o.prefill(step.q, kc, vc, step.block_tables, step.context_lens, step.query_start_loc, step.scale)
    assert torch.equal(out[:14], base[:14]), "future keys leaked into an earlier row"
    assert not torch.equal(out[14:], base[14:]), "later rows must see the changed keys"


def check_prefill_never_reads_unowned_slots(o):
    step = make_prefill_step(query_lens=[1, 15, 17, 40], cached_lens=[0, 16, 3, 256],
                             sharing=[False, False, False, True], dtype=torch.bfloat16,
                             num_q_heads=4, num_kv_heads=2, head_dim=8, seed=27, write_new=False,
                             poison=True)
    out = _pre(o, step)
    assert torch.isfinite(out).all(), "an unowned slot was read"


# ---------------------------------------------------------------------------
# KV-cache write pins
# ---------------------------------------------------------------------------


def check_golden_kv_write(o):
    with open(os.path.join(GOLDEN, "kv_write_example.json")) as f:
        g = json.load(f)
    i16 = lambda x: torch.tensor(x, dtype=torch.int16).view(torch.float16)  # noqa: E731
    kc, vc = i16(g["k_pool_before"]), i16(g["v_pool_before"])
    k2, v2 = o.kv_cache_write(i16(g["new_k"]), i16(g["new_v"]), torch.tensor(g["slot_mapping"]), kc, vc)
    assert k2.view(torch.int16).tolist() == g["k_pool_after"]
    assert v2.view(torch.int16).tolist() == g["v_pool_after"]
    assert kc.view(torch.int16).tolist() == g["k_pool_before"], "inputs must not be modified"


def check_kv_write_scatter(o):
    """After the write, reading each slot returns the row's bits; every other
    byte (NaN payloads included) is unchanged; negative slots write nothing."""
    step = _small_decode([5, 16, 17, 33], seed=28, dtype=torch.bfloat16)
    NB, B = step.num_blocks, step.block_size
    T = 6
    gen = torch.Generator().manual_seed(29)
    newk = torch.randn(T, step.num_kv_heads, step.head_dim, generator=gen).to(torch.bfloat16)
    newv = torch.randn(T, step.num_kv_heads, step.head_dim, generator=gen).to(torch.bfloat16)
    slots = torch.tensor([3, -1, NB * B - 1, 17, -5, 40], dtype=torch.int64)
    k2, v2 = o.kv_cache_write(newk, newv, slots, step.k_cache, step.v_cache)
    fk0 = step.k_cache.view(torch.int16).reshape(NB * B, -1)
    fk2 = k2.view(torch.int16).reshape(NB * B, -1)
    fv2 = v2.view(torch.int16).reshape(NB * B, -1)
    written = set()
    for i, s in enumerate(slots.tolist()):
        if s < 0:
            continue
        written.add(s)
        assert torch.equal(fk2[s], newk[i].view(torch.int16).reshape(-1))
        assert torch.equal(fv2[s], newv[i].view(torch.int16).reshape(-1))
    keep = torch.tensor([s not in written for s in range(NB * B)])
    assert torch.equal(fk2[keep], fk0[keep]), "an unwritten slot changed"


ALL_CHECKS = [
    check_golden_decode,
    check_context_of_one_returns_v,
    check_constant_keys_give_mean_of_v,
    check_zero_scale_gives_mean_of_v,
    check_dominant_key_selects_its_value,
    check_block_permutation_invariance,
    check_brute_force_tiny_pools,
    check_contiguous_pool_matches_sdpa,
    check_gqa_equals_mha_with_repeated_kv,
    check_scale_invariance,
    check_never_reads_unowned_slots,
    check_splitk_merge_equals_unsplit,
    check_splitk_partition_state,
    check_golden_prefill,
    check_prefill_matches_sdpa_bottom_right,
    check_prefill_chunk_invariance,
    check_prefill_rows_equal_decode,
    check_prefill_causality,
    check_prefill_never_reads_unowned_slots,
    check_golden_kv_write,
    check_kv_write_scatter,
]
