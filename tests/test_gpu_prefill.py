"""GPU parity of the MFMA paged prefill (ragged chunks, bottom-right causal
mask, chunks attending to earlier cached chunks, shared-prefix blocks) and of
the full mixed step (KV write, decode rows and prefill rows into one output)
against the fp64 oracle."""

import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DevStep, assert_parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


def run_prefill(pka, ds, out=None):
    step = ds.step
    say(f"prefill {step.name} seed={step.seed} chunks={step.num_prefill} rows={step.num_prefill_rows} "
        f"Hq={step.num_q_heads} Hkv={step.num_kv_heads} D={step.head_dim} {step.dtype} "
        f"qlen={step.meta['prefill_qlen']} cached={step.meta['prefill_cached']}")
    out = pka.paged_attn_prefill(ds.prefill_q, ds.k_cache, ds.v_cache, ds.prefill_block_tables,
                                 ds.prefill_context_lens, ds.query_start_loc, step.scale, step.max_query_len,
                                 int(step.prefill_context_lens.max()), out=out)
    torch.cuda.synchronize()
    return out


def oracle_prefill(step, k_cache=None, v_cache=None, rows=None):
    return oracle.prefill(step.prefill_q, step.k_cache if k_cache is None else k_cache,
                          step.v_cache if v_cache is None else v_cache, step.prefill_block_tables,
                          step.prefill_context_lens, step.query_start_loc, step.scale, rows=rows)


# (q_len, cached) pairs around the 32-key staging tile, the 64-position query
# tile (G = 2) and 16-token KV blocks.
RAGGED = [(1, 0), (31, 0), (32, 0), (33, 1), (63, 15), (64, 16), (65, 17), (127, 0), (128, 100), (129, 0),
          (200, 512), (1, 700)]
SHAPES = [
    (torch.bfloat16, 16, 8, 128),
    (torch.float16, 8, 8, 128),
    (torch.bfloat16, 8, 2, 64),
    (torch.float16, 16, 2, 64),
    (torch.bfloat16, 8, 1, 128),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{str(s[0])[6:]}-{s[1]}q{s[2]}kv-d{s[3]}" for s in SHAPES])
def test_ragged_chunks(pka, shape):
    dtype, hq, hkv, d = shape
    ql = [a for a, _ in RAGGED]
    cl = [b for _, b in RAGGED]
    step = W.make_prefill_step(query_lens=ql, cached_lens=cl, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                               head_dim=d, seed=31, poison=True, write_new=False)
    ds = DevStep(step)
    out = run_prefill(pka, ds)
    assert_parity(out, oracle_prefill(step), dtype, f"ragged prefill {shape}", weights_rounded=True)


def test_many_chunks_grid_order(pka):
    """More chunks (300) than the kernel's heavy-first item ordering takes
    (256): every workgroup falls back to grid order (query tile, split) and
    the batch must still be covered exactly once.  Chunks of 1-40 rows after
    0-300 cached tokens, so their ends fall anywhere inside KV blocks and key
    tiles."""
    ql = [1 + (7 * i) % 40 for i in range(300)]
    cl = [(37 * i) % 301 for i in range(300)]
    step = W.make_prefill_step(query_lens=ql, cached_lens=cl, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                               head_dim=128, seed=38, poison=True, write_new=False)
    ds = DevStep(step)
    out = run_prefill(pka, ds)
    assert_parity(out, oracle_prefill(step), step.dtype, "300-chunk prefill (grid order)", weights_rounded=True)


@pytest.mark.parametrize("shape", [(torch.bfloat16, 16, 8, 128), (torch.float16, 8, 8, 64)],
                         ids=["bf16-16q8kv-d128", "fp16-8q8kv-d64"])
def test_long_context_splits(pka, shape):
    """Query tiles whose visible keys cross key-split boundaries: a tile
    ending exactly at the first boundary, one ending one key past it, one
    ending exactly at the second, several splits, and a single row after a
    7,679-token prefix (which fixes the longest context and so, with the
    chunk sizes, the split length the launch picks)."""
    dtype, hq, hkv, d = shape
    ql = [64, 65, 128, 1, 300, 17]
    keys = pka.prefill_split_keys(len(ql), sum(ql), hq, hkv, d, 7680)
    say(f"split length {keys} keys")
    bq = 128 // (hq // hkv)  # query positions per tile
    # first tile of chunk 0 ends at keys, of chunk 1 at keys + 1; chunk 5 ends at 2 * keys
    cached = [keys - min(64, bq), keys + 1 - min(65, bq), 3000, 7679, 2500, 2 * keys - 17]
    assert all(0 <= c and c + q <= 7680 for c, q in zip(cached, ql))
    step = W.make_prefill_step(query_lens=ql, cached_lens=cached,
                               dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, seed=36, poison=True,
                               write_new=False)
    ds = DevStep(step)
    out = run_prefill(pka, ds)
    assert_parity(out, oracle_prefill(step), dtype, f"long-context splits {shape}", weights_rounded=True)


def test_workspace_reuse_across_calls(pka):
    """One workspace serves consecutive calls (same bits every time)."""
    step = W.make_prefill_step(query_lens=[200, 64, 1], cached_lens=[3000, 1500, 5000], dtype=torch.bfloat16,
                               num_q_heads=16, num_kv_heads=8, head_dim=128, seed=37, poison=True, write_new=False)
    ds = DevStep(step)
    mcl = int(step.prefill_context_lens.max())
    need = pka.prefill_workspace_bytes(step.num_prefill, step.num_prefill_rows, 16, 8, 128, mcl)
    assert need > 0
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device="cuda")  # garbage-filled: contents are scratch
    ref = oracle_prefill(step)
    outs = []
    for call in range(3):
        say(f"prefill with a reused workspace, call {call}")
        out = pka.paged_attn_prefill(ds.prefill_q, ds.k_cache, ds.v_cache, ds.prefill_block_tables,
                                     ds.prefill_context_lens, ds.query_start_loc, step.scale, step.max_query_len, mcl,
                                     workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out, ref, step.dtype, f"reused workspace call {call}", weights_rounded=True)
        outs.append(out.cpu().view(torch.int16))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_shared_prefix_chunks(pka):
    """Chunks whose tables share one 256-token prefix (refcounted blocks),
    each starting right after the prefix or later."""
    step = W.make_prefill_step(query_lens=[100, 37, 256, 1], cached_lens=[256, 256, 512, 300],
                               sharing=[True, True, True, False], dtype=torch.bfloat16, num_q_heads=16,
                               num_kv_heads=8, head_dim=128, seed=32, poison=True, write_new=False)
    assert step.refcount.max() == 3
    ds = DevStep(step)
    out = run_prefill(pka, ds)
    assert_parity(out, oracle_prefill(step), step.dtype, "shared-prefix prefill", weights_rounded=True)


def test_write_then_prefill(pka):
    """The chunk's own K/V arrive through the KV write right before attention."""
    step = W.make_prefill_step(query_lens=[70, 5], cached_lens=[33, 0], dtype=torch.bfloat16, num_q_heads=16,
                               num_kv_heads=8, head_dim=128, seed=33, poison=True, write_new=True)
    ds = DevStep(step)
    pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
    kc, vc = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, step.k_cache, step.v_cache)
    out = run_prefill(pka, ds)
    assert_parity(out, oracle_prefill(step, kc, vc), step.dtype, "write then prefill", weights_rounded=True)


@pytest.mark.parametrize("seed", [0, 1])
def test_config5_mixed_step_full(pka, seed):
    """The measured mixed step at full size: KV write of all 2,048 new rows,
    then decode into out[:64] and prefill into out[64:] of one output tensor."""
    step = W.config_5(seed=seed, poison=True)
    ds = DevStep(step)
    say(f"config5 seed {seed}: kv write {step.slot_mapping.numel()} rows; chunks qlen={step.meta['prefill_qlen']} "
        f"cached={step.meta['prefill_cached']}")
    pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
    out = torch.full_like(ds.q, float("nan"))
    nd = step.num_decode
    pka.paged_attn_decode(ds.decode_q, ds.k_cache, ds.v_cache, ds.decode_block_tables, ds.decode_context_lens,
                          step.scale, int(step.decode_context_lens.max()), out=out[:nd])
    pka.paged_attn_prefill(ds.prefill_q, ds.k_cache, ds.v_cache, ds.prefill_block_tables, ds.prefill_context_lens,
                           ds.query_start_loc, step.scale, step.max_query_len, int(step.prefill_context_lens.max()),
                           out=out[nd:])
    torch.cuda.synchronize()
    kc, vc = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, step.k_cache, step.v_cache)
    assert torch.equal(ds.k_cache.cpu().view(torch.int16), kc.view(torch.int16))
    ref_dec = oracle.decode(step.decode_q, kc, vc, step.decode_block_tables, step.decode_context_lens, step.scale)
    assert_parity(out[:nd], ref_dec, step.dtype, f"config5 seed {seed} decode rows")
    ref_pre = oracle_prefill(step, kc, vc)
    assert_parity(out[nd:], ref_pre, step.dtype, f"config5 seed {seed} prefill rows", weights_rounded=True)


def test_single_row_chunk_matches_decode_rows(pka):
    """A one-row chunk is a decode: both kernels against the oracle."""
    step = W.make_prefill_step(query_lens=[1, 1, 1], cached_lens=[0, 255, 1999], dtype=torch.bfloat16,
                               num_q_heads=16, num_kv_heads=8, head_dim=128, seed=34, poison=True, write_new=False)
    ds = DevStep(step)
    out = run_prefill(pka, ds)
    ref = oracle.decode(step.q, step.k_cache, step.v_cache, step.block_tables, step.context_lens, step.scale)
    assert_parity(out, ref, step.dtype, "one-row chunks vs decode oracle", weights_rounded=True)
    dec = pka.paged_attn_decode_v1(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.context_lens, step.scale)
    torch.cuda.synchronize()
    assert_parity(dec, ref, step.dtype, "decode kernel on the same rows")


def test_prefill_repeat_and_placement_bit_identity(pka):
    step = W.make_prefill_step(query_lens=[90, 17, 300], cached_lens=[40, 500, 0], dtype=torch.bfloat16,
                               num_q_heads=16, num_kv_heads=8, head_dim=128, seed=35, poison=True, write_new=False)
    ds = DevStep(step)
    a = run_prefill(pka, ds)
    b = run_prefill(pka, ds)
    assert torch.equal(a.cpu().view(torch.int16), b.cpu().view(torch.int16)), "repeat run differs"
    perm = torch.randperm(step.num_blocks, generator=torch.Generator().manual_seed(2))
    kc = torch.empty_like(step.k_cache)
    vc = torch.empty_like(step.v_cache)
    kc[perm] = step.k_cache
    vc[perm] = step.v_cache
    step.k_cache, step.v_cache = kc, vc
    step.block_tables = perm[step.block_tables.long()].to(torch.int32)
    c = run_prefill(pka, DevStep(step))
    assert torch.equal(a.cpu().view(torch.int16), c.cpu().view(torch.int16)), "block relabelling changed bits"


# Block sizes 8 and 32 (a 32-key staging tile then spans four or one blocks),
# and head size 256 (eight wavefronts of 16 q-rows per query tile).
GENERAL = [
    (torch.bfloat16, 16, 8, 128, 8),
    (torch.bfloat16, 16, 8, 128, 32),
    (torch.float16, 8, 2, 64, 8),
    (torch.float16, 8, 8, 64, 32),
    (torch.bfloat16, 16, 8, 256, 16),
    (torch.float16, 8, 4, 256, 32),
    (torch.bfloat16, 8, 1, 256, 8),
]


@pytest.mark.parametrize("shape", GENERAL, ids=[f"{str(s[0])[6:]}-{s[1]}q{s[2]}kv-d{s[3]}-b{s[4]}" for s in GENERAL])
def test_general_shapes(pka, shape):
    dtype, hq, hkv, d, bs = shape
    step = W.make_prefill_step(query_lens=[1, 31, 33, 64, 129, 200, 17], cached_lens=[0, 7, 1, 100, 40, 1100, 2047],
                               dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, seed=38,
                               poison=True, write_new=False)
    ds = DevStep(step)
    out = run_prefill(pka, ds)
    assert_parity(out, oracle_prefill(step), dtype, f"prefill shape {shape}", weights_rounded=True)


@pytest.mark.parametrize("heads", [(16, 8, 128, 16), (8, 4, 256, 8), (8, 4, 128, 16)],
                         ids=["16q8kv-d128", "8q4kv-d256-b8", "8q4kv-d128"])
def test_long_prefill_bench_size_sampled_rows(pka, heads):
    """The long-prefill workload at the size and in the launch configuration
    the benchmark times (4 chunks of 2,048 rows after 6,144 cached tokens,
    bf16, 16q/8kv, head_dim 128, workspace sized by the library), checked on
    sampled rows: both ends of every chunk, rows around query-tile (64
    positions) boundaries, and random rows.  Also at 8q/4kv: unsplit at head
    size 256 (one workgroup per compute unit: 528 items are two rounds), split
    in two at head size 128."""
    hq, hkv, d, bs = heads
    ql, cached = [2048] * 4, [6144] * 4
    step = W.make_prefill_step(query_lens=ql, cached_lens=cached, dtype=torch.bfloat16, num_q_heads=hq,
                               num_kv_heads=hkv, head_dim=d, block_size=bs, seed=0, poison=True, write_new=False)
    ds = DevStep(step)
    Hq, D, Hkv = step.num_q_heads, step.head_dim, step.num_kv_heads
    mcl = int(step.prefill_context_lens.max())
    ws = torch.empty(max(1, pka.prefill_workspace_bytes(step.num_prefill, step.num_prefill_rows, Hq, Hkv, D, mcl)),
                     dtype=torch.uint8, device="cuda")
    say(f"long prefill at bench size: split length {pka.prefill_split_keys(4, 8192, Hq, Hkv, D, mcl)} keys")
    out = pka.paged_attn_prefill(ds.prefill_q, ds.k_cache, ds.v_cache, ds.prefill_block_tables,
                                 ds.prefill_context_lens, ds.query_start_loc, step.scale, step.max_query_len, mcl,
                                 out=None, workspace=ws)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(5)
    rows = set()
    for j in range(4):
        b = j * 2048
        rows.update(b + r for r in (0, 1, 63, 64, 65, 127, 128, 1023, 1024, 2046, 2047))
        rows.update((b + torch.randint(0, 2048, (6,), generator=g)).tolist())
    rows = sorted(rows)
    ref = oracle_prefill(step, rows=rows)
    assert_parity(out.cpu()[rows], ref[rows], step.dtype, f"long prefill bench size {heads}, {len(rows)} sampled rows",
                  weights_rounded=True)
