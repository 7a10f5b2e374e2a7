"""GPU parity of paged decode (single pass, split-K + reduce, dispatcher)
against the fp64 oracle, on the measured configs at full size and on edge
cases.  Pools are NaN-poisoned wherever no sequence owns a slot, so any stray
read shows up as a non-finite output."""

import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import TOL, DevStep, assert_parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


def oracle_decode(step, seqs=None, k_cache=None, v_cache=None):
    return oracle.decode(step.decode_q, step.k_cache if k_cache is None else k_cache,
                         step.v_cache if v_cache is None else v_cache, step.decode_block_tables,
                         step.decode_context_lens, step.scale, seqs=seqs)


def run_decode(pka, ds, variant, max_ctx=None):
    step = ds.step
    S, Hq, D = ds.decode_q.shape
    max_ctx = int(step.decode_context_lens.max()) if max_ctx is None else max_ctx
    say(f"decode {variant} {step.name} seed={step.seed} S={S} Hq={Hq} Hkv={step.num_kv_heads} D={D} "
        f"{step.dtype} max_ctx={max_ctx}")
    args = (ds.decode_q, ds.k_cache, ds.v_cache, ds.decode_block_tables, ds.decode_context_lens, step.scale)
    if variant == "auto":
        out = pka.paged_attn_decode(*args, max_context_len=max_ctx)
    elif variant == "v1":
        out = pka.paged_attn_decode_v1(*args)
    elif variant == "v2":
        bufs = pka.splitk_buffers(S, Hq, D, max_ctx, ds.q.device)
        pka.paged_attn_decode_splitk(*args, *bufs)
        out = torch.empty_like(ds.decode_q)
        pka.paged_attn_splitk_reduce(*bufs, ds.decode_context_lens, out)
    else:
        raise ValueError(variant)
    torch.cuda.synchronize()
    return out


VARIANTS = ["auto", "v1", "v2"]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_config1_single_request_fp16(pka, seed, variant):
    step = W.config_1(seed=seed, poison=True)
    ds = DevStep(step)
    out = run_decode(pka, ds, variant)
    assert_parity(out, oracle_decode(step), step.dtype, f"config1 seed {seed} {variant}")


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("ctx", [128, 1024, 4096])
def test_config2_context_sweep_fp16(pka, ctx, variant):
    step = W.config_2(ctx, seed=0, poison=True)
    ds = DevStep(step)
    out = run_decode(pka, ds, variant)
    assert_parity(out, oracle_decode(step), step.dtype, f"config2 ctx {ctx} {variant}")


def test_config3_write_then_decode_full(pka):
    """The measured step at full size: KV write of 256 rows, then dispatched
    decode over 256 sequences reading the rows just written."""
    step = W.config_3(seed=0, poison=True)
    ds = DevStep(step)
    say("config3 kv_cache_write 256 rows")
    pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
    torch.cuda.synchronize()
    kc, vc = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, step.k_cache, step.v_cache)
    assert torch.equal(ds.k_cache.cpu().view(torch.int16), kc.view(torch.int16)), "K pool differs bitwise"
    assert torch.equal(ds.v_cache.cpu().view(torch.int16), vc.view(torch.int16)), "V pool differs bitwise"
    ref = oracle_decode(step, k_cache=kc, v_cache=vc)
    for variant in VARIANTS:
        out = run_decode(pka, ds, variant)
        assert_parity(out, ref, step.dtype, f"config3 full {variant}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_config4_long_context_full(pka, variant):
    step = W.config_4(seed=0, poison=True)
    ds = DevStep(step)
    out = run_decode(pka, ds, variant)
    assert_parity(out, oracle_decode(step), step.dtype, f"config4 {variant}")


EDGE_CTX = [1, 2, 15, 16, 17, 31, 255, 256, 257, 511, 512, 513, 1000]
SHAPES = [
    (torch.float16, 2, 2, 64),
    (torch.bfloat16, 16, 8, 128),
    (torch.float16, 8, 4, 128),
    (torch.bfloat16, 4, 1, 64),
    (torch.bfloat16, 8, 1, 128),
    (torch.float16, 4, 4, 128),
    (torch.bfloat16, 16, 4, 64),
]


@pytest.mark.parametrize("variant", ["v1", "v2"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"{str(s[0])[6:]}-{s[1]}q{s[2]}kv-d{s[3]}" for s in SHAPES])
def test_edge_context_lengths(pka, shape, variant):
    dtype, hq, hkv, d = shape
    step = W.make_decode_step(context_lens=EDGE_CTX, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                              seed=7, poison=True, pool_factor=1.3)
    ds = DevStep(step)
    out = run_decode(pka, ds, variant)
    assert_parity(out, oracle_decode(step), dtype, f"edge lengths {shape} {variant}")


@pytest.mark.parametrize("variant", ["v1", "auto"])
@pytest.mark.parametrize("num_seqs", [600, 1100])
def test_many_sequences_longest_first(pka, num_seqs, variant):
    """The single pass runs sequences longest first (up to 1,024 sequences;
    grid order above): every sequence must still be computed exactly once,
    whatever its rank - lengths spread over many buckets, with ties, a few
    very long contexts and some of one token."""
    g = torch.Generator().manual_seed(num_seqs)
    ctx = torch.randint(1, 200, (num_seqs,), generator=g)
    ctx[torch.randint(0, num_seqs, (12,), generator=g)] = 1
    ctx[torch.randint(0, num_seqs, (6,), generator=g)] = 1500
    ctx[::97] = 64  # ties
    step = W.make_decode_step(context_lens=ctx.tolist(), dtype=torch.float16, num_q_heads=4, num_kv_heads=2,
                              head_dim=64, seed=num_seqs, poison=True)
    ds = DevStep(step)
    out = run_decode(pka, ds, variant, max_ctx=int(ctx.max()))
    assert_parity(out, oracle_decode(step), step.dtype, f"{num_seqs} sequences {variant}")


def test_splitk_partition_state_matches_oracle(pka):
    step = W.make_decode_step(context_lens=[1, 255, 256, 257, 700, 2049], dtype=torch.bfloat16, num_q_heads=16,
                              num_kv_heads=8, head_dim=128, seed=8, poison=True)
    ds = DevStep(step)
    S, Hq, D = step.decode_q.shape
    bufs = pka.splitk_buffers(S, Hq, D, step.max_context_len, ds.q.device)
    for b in bufs:
        b.fill_(float("nan"))
    say("splitk partition state vs oracle")
    pka.paged_attn_decode_splitk(ds.decode_q, ds.k_cache, ds.v_cache, ds.decode_block_tables, ds.decode_context_lens,
                                 step.scale, *bufs)
    torch.cuda.synchronize()
    m, l, po, npart = oracle.decode_partitions(step.decode_q, step.k_cache, step.v_cache, step.decode_block_tables,
                                               step.decode_context_lens, step.scale, 256)
    tmp_out, max_logits, exp_sums = (b.cpu().double() for b in bufs)
    for s in range(S):
        P = int(npart[s])
        assert torch.isfinite(max_logits[s, :, :P]).all()
        assert torch.isnan(max_logits[s, :, P:]).all(), "partition past the end was written"
        em = (max_logits[s, :, :P] - m[s, :, :P]).abs().max().item()
        el = ((exp_sums[s, :, :P] - l[s, :, :P]).abs() / l[s, :, :P]).max().item()
        eo = (tmp_out[s, :, :P] - po[s, :, :P]).abs().max().item()
        say(f"seq {s} P={P}: max-logit err {em:.2e}, exp-sum rel err {el:.2e}, partial-out err {eo:.2e}")
        assert em < 1e-4 and el < 1e-4 and eo < 1e-4


@pytest.mark.parametrize("variant", ["v1", "v2", "auto"])
def test_block_placement_bit_identity(pka, variant):
    """Relabelling physical blocks (moving contents and table entries
    together) must not change a single output bit: the summation order depends
    only on logical positions."""
    step = W.make_decode_step(context_lens=[17, 300, 1025, 2000], dtype=torch.bfloat16, num_q_heads=16,
                              num_kv_heads=8, head_dim=128, seed=9, poison=True)
    ds = DevStep(step)
    base = run_decode(pka, ds, variant)
    perm = torch.randperm(step.num_blocks, generator=torch.Generator().manual_seed(1))
    kc = torch.empty_like(step.k_cache)
    vc = torch.empty_like(step.v_cache)
    kc[perm] = step.k_cache
    vc[perm] = step.v_cache
    step.k_cache, step.v_cache = kc, vc
    step.block_tables = perm[step.block_tables.long()].to(torch.int32)
    ds2 = DevStep(step)
    out = run_decode(pka, ds2, variant)
    assert torch.equal(out.cpu().view(torch.int16), base.cpu().view(torch.int16))


@pytest.mark.parametrize("variant", ["v1", "v2", "auto"])
def test_repeat_runs_bit_identical(pka, variant):
    step = W.make_decode_step(context_lens=[5, 513, 1999, 64], dtype=torch.float16, num_q_heads=8, num_kv_heads=4,
                              head_dim=128, seed=10, poison=True)
    ds = DevStep(step)
    a = run_decode(pka, ds, variant)
    b = run_decode(pka, ds, variant)
    assert torch.equal(a.cpu().view(torch.int16), b.cpu().view(torch.int16))


def test_empty_batch_is_noop(pka):
    step = W.make_decode_step(context_lens=[16], dtype=torch.bfloat16, seed=11)
    ds = DevStep(step)
    q0 = ds.decode_q[:0]
    say("decode with zero sequences")
    out = pka.paged_attn_decode_v1(q0, ds.k_cache, ds.v_cache, ds.decode_block_tables[:0], ds.decode_context_lens[:0],
                                   step.scale)
    torch.cuda.synchronize()
    assert out.shape[0] == 0


def test_tolerances_are_the_stated_ones():
    assert TOL[torch.float16] == 2e-3 and TOL[torch.bfloat16] == 1.5e-2


# Block sizes other than 16 and head size 256 (mini_engine, "Roadmap":
# generalising the kernels beyond one head shape).  (dtype, Hq, Hkv, D, block)
GENERAL = [
    (torch.bfloat16, 16, 8, 128, 8),
    (torch.bfloat16, 16, 8, 128, 32),
    (torch.float16, 2, 2, 64, 32),
    (torch.float16, 8, 2, 64, 8),
    (torch.bfloat16, 8, 8, 256, 16),
    (torch.bfloat16, 16, 2, 256, 8),
    (torch.float16, 4, 1, 256, 32),
    # groups of eight (q in LDS, two-load tiles) and 32-slot blocks of head
    # size 256 (four tiles per block)
    (torch.bfloat16, 16, 2, 128, 16),
    (torch.bfloat16, 32, 4, 128, 32),
    (torch.float16, 16, 2, 256, 32),
    (torch.bfloat16, 8, 4, 256, 32),
    # group 4 at head size 256 with 32-slot blocks, bf16 (one unit in flight
    # on the matrix cores; the partition-only form under v2)
    (torch.bfloat16, 32, 8, 256, 32),
]


@pytest.mark.parametrize("variant", ["v1", "v2"])
@pytest.mark.parametrize("shape", GENERAL, ids=[f"{str(s[0])[6:]}-{s[1]}q{s[2]}kv-d{s[3]}-b{s[4]}" for s in GENERAL])
def test_general_block_and_head_sizes(pka, shape, variant):
    """Write-then-decode over ragged contexts (around block, partition and
    window boundaries) for each block size / head size."""
    dtype, hq, hkv, d, bs = shape
    ctx = [1, bs - 1, bs, bs + 1, 255, 256, 257, 1000, 64 * bs + 3]
    step = W.make_decode_step(context_lens=ctx, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                              block_size=bs, seed=9, poison=True, write_new=True)
    ds = DevStep(step)
    pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
    kc, vc = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, step.k_cache, step.v_cache)
    torch.cuda.synchronize()
    assert torch.equal(ds.k_cache.cpu().view(torch.int16), kc.view(torch.int16)), "KV write not bit-exact"
    assert torch.equal(ds.v_cache.cpu().view(torch.int16), vc.view(torch.int16)), "KV write not bit-exact"
    out = run_decode(pka, ds, variant)
    assert_parity(out, oracle_decode(step, k_cache=kc, v_cache=vc), dtype, f"general {shape} {variant}")


@pytest.mark.parametrize("num_seqs,hkv", [(40, 8), (64, 8), (150, 2), (33, 8)])
def test_one_round_grid_pairing(pka, num_seqs, hkv):
    """Grids of more (sequence, KV head) workgroups than compute units but at
    most two per unit reverse the order of the rows that take a second slot
    (long sequences paired with short ones): every sequence must still be
    computed exactly once, whatever its rank."""
    cus = pka.device_cu_count()
    say(f"one-round pairing: {num_seqs} seqs x {hkv} KV heads on {cus} CUs")
    g = torch.Generator().manual_seed(num_seqs * hkv)
    ctx = torch.randint(1, 2049, (num_seqs,), generator=g)
    ctx[::7] = 1
    step = W.make_decode_step(context_lens=ctx.tolist(), dtype=torch.bfloat16, num_q_heads=2 * hkv, num_kv_heads=hkv,
                              head_dim=128, seed=num_seqs, poison=True)
    ds = DevStep(step)
    for variant in ("v1", "auto"):
        out = run_decode(pka, ds, variant)
        assert_parity(out, oracle_decode(step), step.dtype, f"pairing {num_seqs}x{hkv} {variant}")


@pytest.mark.parametrize("variant", VARIANTS)
def test_fp16_long_context_reduce_loop(pka, variant):
    """fp16 (tolerance 2e-3) at 6,400+ tokens: 26-40 partitions per sequence,
    so the reduce's unrolled partition loop and the single-launch merge run
    at the tighter fp16 bound, next to shorter sequences of the same batch."""
    step = W.make_decode_step(context_lens=[6401, 10240, 777, 7000], dtype=torch.float16, num_q_heads=8,
                              num_kv_heads=4, head_dim=128, seed=12, poison=True)
    ds = DevStep(step)
    out = run_decode(pka, ds, variant)
    assert_parity(out, oracle_decode(step), step.dtype, f"fp16 6,400+ tokens {variant}")


@pytest.mark.parametrize("variant", ["v2", "auto"])
@pytest.mark.parametrize("shape", [(torch.float16, 2, 2, 64, [262400, 300]),
                                   (torch.bfloat16, 16, 8, 128, [140000, 300]),
                                   (torch.bfloat16, 4, 2, 128, [140000]),
                                   (torch.bfloat16, 16, 2, 128, [40000])],
                         ids=["fp16-2q2kv-d64-262400", "bf16-16q8kv-d128-140000", "bf16-4q2kv-d128-140000",
                              "bf16-16q2kv-d128-40000"])
def test_more_partitions_than_one_merge_pass(pka, shape, variant):
    """Long contexts.  The two-launch reduce stages 1,024 partitions per
    pass, so 1,025 partitions (262,400 tokens) take two.  The single-launch
    path merges one state per workgroup, 8 x (threads per 4-dim column) states
    per pass: a lone 140,000-token sequence with 2 KV heads leaves 69
    workgroup states at G = 2 (passes of 64), and 40,000 tokens at G = 8 leave
    20 (passes of 16).  Short sequences ride beside the long ones."""
    dtype, hq, hkv, d, ctx = shape
    step = W.make_decode_step(context_lens=ctx, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                              seed=13, poison=True, pool_factor=1.02)
    ds = DevStep(step)
    out = run_decode(pka, ds, variant)
    assert_parity(out, oracle_decode(step), dtype, f"{ctx[0]} tokens {variant}")


def test_single_launch_splitk_workspace_reuse(pka):
    """The single-launch split-K leaves its arrival counters at zero: one
    workspace (zeroed once) serves calls of different sizes in a row, its
    partial-result region filled with garbage before each, and the counter
    header reads zero after every call."""
    ws = pka.splitk_workspace(8, 16, 128, 9000, "cuda")
    header = 65536
    cases = [([9000, 4000, 300, 8192], 8), ([5000], 1), ([7000, 6000, 1, 256, 257, 4097, 8999, 2000], 8),
             ([3000, 9000], 2)]
    for i, (ctx, n) in enumerate(cases):
        step = W.make_decode_step(context_lens=ctx, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                                  head_dim=128, seed=20 + i, poison=True)
        ds = DevStep(step)
        assert pka.decode_choose_variant(n, 8, max(ctx)) == 2
        ws[header:].fill_(0xFF)
        say(f"workspace reuse call {i}: contexts {ctx}")
        out = pka.paged_attn_decode(ds.decode_q, ds.k_cache, ds.v_cache, ds.decode_block_tables,
                                    ds.decode_context_lens, step.scale, max(ctx), workspace=ws)
        torch.cuda.synchronize()
        assert_parity(out, oracle_decode(step), step.dtype, f"workspace reuse call {i}")
        assert int(ws[:header].count_nonzero()) == 0, f"call {i} left a counter non-zero"


def test_splitk_two_launch_fallback_many_pairs(pka):
    """More (sequence, KV head) pairs than the counter header holds (2,100 x
    8 > 16,384) with a context long enough for split-K: the dispatcher takes
    the partition pass + reduce in two launches."""
    g = torch.Generator().manual_seed(2100)
    ctx = torch.randint(1, 400, (2100,), generator=g)
    ctx[::300] = 4600
    step = W.make_decode_step(context_lens=ctx.tolist(), dtype=torch.bfloat16, num_q_heads=8, num_kv_heads=8,
                              head_dim=64, seed=14, poison=True)
    assert pka.decode_choose_variant(2100, 8, int(ctx.max())) == 2
    ds = DevStep(step)
    out = run_decode(pka, ds, "auto")
    assert_parity(out, oracle_decode(step), step.dtype, "2,100 x 8 pairs, two-launch split-K")
