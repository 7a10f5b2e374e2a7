"""GPU parity of the decode step with the KV-cache write folded in
(pka_paged_attn_decode_append): the pools must equal the oracle's scatter of
the new rows bit for bit, and the output must equal the oracle's decode over
the written pools.  The slots about to be written hold NaN beforehand, so a
kernel that read a new token back from the cache instead of from its
registers would produce NaN."""

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


def check_append(pka, step, what, max_ctx=None):
    ds = DevStep(step)
    S, Hq, D = step.decode_q.shape
    assert step.new_k.shape[0] == S, "one new row per sequence"
    max_ctx = int(step.decode_context_lens.max()) if max_ctx is None else max_ctx
    variant = pka.decode_choose_variant(S, step.num_kv_heads, max_ctx)
    say(f"decode_append {what} S={S} Hq={Hq} Hkv={step.num_kv_heads} D={D} block={step.block_size} "
        f"{step.dtype} max_ctx={max_ctx} variant={variant}")
    out = pka.paged_attn_decode_append(ds.decode_q, ds.new_k, ds.new_v, ds.k_cache, ds.v_cache,
                                       ds.decode_block_tables, ds.decode_context_lens, step.scale,
                                       max_context_len=max_ctx)
    torch.cuda.synchronize()
    kc, vc = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, step.k_cache, step.v_cache)
    assert torch.equal(ds.k_cache.cpu().view(torch.int16), kc.view(torch.int16)), f"{what}: K pool differs bitwise"
    assert torch.equal(ds.v_cache.cpu().view(torch.int16), vc.view(torch.int16)), f"{what}: V pool differs bitwise"
    ref = oracle.decode(step.decode_q, kc, vc, step.decode_block_tables, step.decode_context_lens, step.scale)
    assert_parity(out, ref, step.dtype, f"decode_append {what}")
    return variant


@pytest.mark.parametrize("seed", [0, 1])
def test_config3_append_full(pka, seed):
    """The measured decode step at full size (256 sequences, single pass)."""
    assert check_append(pka, W.config_3(seed=seed, poison=True), f"config3 seed {seed}") == 1


# (dtype, Hq, Hkv, D, block): the shapes of the decode tests, every block size
# and head size.
SHAPES = [
    (torch.bfloat16, 16, 8, 128, 16),
    (torch.float16, 2, 2, 64, 16),
    (torch.float16, 8, 4, 128, 16),
    (torch.bfloat16, 16, 8, 128, 8),
    (torch.bfloat16, 16, 8, 128, 32),
    (torch.float16, 8, 2, 64, 8),
    (torch.bfloat16, 8, 8, 256, 16),
    (torch.float16, 4, 1, 256, 32),
    # groups of eight and 32-slot blocks of head size 256: blocks streamed
    # as several tiles, the appended token in any of them
    (torch.bfloat16, 16, 2, 128, 16),
    (torch.float16, 16, 2, 256, 32),
    (torch.bfloat16, 8, 4, 256, 32),
]
IDS = [f"{str(s[0])[6:]}-{s[1]}q{s[2]}kv-d{s[3]}-b{s[4]}" for s in SHAPES]


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_edge_lengths_split_path(pka, shape):
    """A few sequences with long contexts: the dispatcher takes split-K, and
    the appended token sits in the last partition - first, last and middle
    row of a block, a one-token context, partition boundaries."""
    dtype, hq, hkv, d, bs = shape
    ctx = [1, 2, bs - 1, bs, bs + 1, 255, 256, 257, 513, 1000, 64 * bs + 3]
    step = W.make_decode_step(context_lens=ctx, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                              block_size=bs, seed=21, poison=True, write_new=True)
    assert check_append(pka, step, f"edge {shape}") == 2


@pytest.mark.parametrize("shape", SHAPES[:6], ids=IDS[:6])
def test_many_sequences_single_pass(pka, shape):
    """Enough (sequence, KV head) workgroups for the single pass (longest
    first), ragged lengths with ties and one-token contexts."""
    dtype, hq, hkv, d, bs = shape
    n = max(600, 1200 // hkv)
    g = torch.Generator().manual_seed(n + bs)
    ctx = torch.randint(1, 400, (n,), generator=g)
    ctx[::53] = 1
    ctx[::89] = bs
    step = W.make_decode_step(context_lens=ctx.tolist(), dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                              block_size=bs, seed=n, poison=True, write_new=True)
    assert check_append(pka, step, f"many {shape}") == 1


def test_append_matches_write_then_decode_bitwise(pka):
    """The fused step and the two separate launches compute the same
    attention in the same order: identical output bits."""
    step = W.config_3(seed=2, poison=True, num_seqs=300)
    a = DevStep(step)
    b = DevStep(step)
    S = step.decode_q.shape[0]
    max_ctx = int(step.decode_context_lens.max())
    say(f"append vs write + decode, {S} sequences")
    out_f = pka.paged_attn_decode_append(a.decode_q, a.new_k, a.new_v, a.k_cache, a.v_cache, a.decode_block_tables,
                                         a.decode_context_lens, step.scale, max_context_len=max_ctx)
    pka.kv_cache_write(b.new_k, b.new_v, b.slot_mapping, b.k_cache, b.v_cache)
    out_s = pka.paged_attn_decode(b.decode_q, b.k_cache, b.v_cache, b.decode_block_tables, b.decode_context_lens,
                                  step.scale, max_context_len=max_ctx)
    torch.cuda.synchronize()
    assert torch.equal(out_f.cpu().view(torch.int16), out_s.cpu().view(torch.int16))
    assert torch.equal(a.k_cache.cpu().view(torch.int16), b.k_cache.cpu().view(torch.int16))
    assert torch.equal(a.v_cache.cpu().view(torch.int16), b.v_cache.cpu().view(torch.int16))


def test_append_rejects_bad_rows(pka):
    step = W.make_decode_step(context_lens=[5, 9], dtype=torch.bfloat16, seed=3, write_new=True)
    ds = DevStep(step)
    say("decode_append argument checks")
    with pytest.raises(ValueError):
        pka.paged_attn_decode_append(ds.decode_q, ds.new_k[:1], ds.new_v[:1], ds.k_cache, ds.v_cache,
                                     ds.decode_block_tables, ds.decode_context_lens, step.scale, max_context_len=9)
    with pytest.raises(ValueError):
        pka.paged_attn_decode_append(ds.decode_q, ds.new_k.half(), ds.new_v, ds.k_cache, ds.v_cache,
                                     ds.decode_block_tables, ds.decode_context_lens, step.scale, max_context_len=9)


def test_append_empty_batch_is_noop(pka):
    step = W.make_decode_step(context_lens=[16], dtype=torch.bfloat16, seed=11, write_new=True)
    ds = DevStep(step)
    k0 = ds.k_cache.clone()
    say("decode_append with zero sequences")
    out = pka.paged_attn_decode_append(ds.decode_q[:0], ds.new_k[:0], ds.new_v[:0], ds.k_cache, ds.v_cache,
                                       ds.decode_block_tables[:0], ds.decode_context_lens[:0], step.scale,
                                       max_context_len=16)
    torch.cuda.synchronize()
    assert out.shape[0] == 0
    assert torch.equal(ds.k_cache.view(torch.int16), k0.view(torch.int16)), "an empty batch wrote to the pool"
