"""GPU parity of the rotary table and the fused RoPE + KV-cache write against
the fp64 oracle.  Rotated values are compared in units of the output type's
spacing (the kernel rotates in fp32 and rounds once, the oracle in fp64):
at most one unit apart, and most of them identical; V and every byte of the
pool outside the written slots must be bit-exact."""


import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import assert_parity, say

pytestmark = pytest.mark.gpu

THETA = 1e6  # Qwen3's rotary base


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


def ulps(gpu: torch.Tensor, ref: torch.Tensor) -> torch.Tensor:
    """|gpu - ref| in units of the spacing of gpu's type at ref's magnitude."""
    mant = {torch.bfloat16: 7, torch.float16: 10}[gpu.dtype]
    g = gpu.cpu().double()
    r = ref.double()
    mag = r.abs().clamp_min(2.0 ** -14)
    spacing = torch.exp2(torch.floor(torch.log2(mag)) - mant)
    return (g - r).abs() / spacing


def check_rotated(gpu, ref64, ref_rounded, what, max_ulps=1.0, min_exact=0.95):
    """gpu within max_ulps of the fp64 rotation, and mostly the same bits as
    the oracle's single rounding of it."""
    u = ulps(gpu, ref64)
    assert torch.isfinite(gpu.cpu().float()).all(), f"{what}: non-finite output"
    worst = float(u.max())
    exact = float((gpu.cpu().view(torch.int16) == ref_rounded.view(torch.int16)).double().mean())
    say(f"{what}: max {worst:.2f} ulp, {100 * exact:.2f}% identical")
    assert worst <= max_ulps, f"{what}: {worst} ulps"
    assert exact >= min_exact, f"{what}: only {exact:.3f} identical"


def test_table_matches_oracle_angles(pka):
    max_pos, D = 32768, 128
    say(f"rope table {max_pos} x {D}, theta {THETA}")
    table = pka.rope_table(max_pos, D, THETA, "cuda")
    torch.cuda.synchronize()
    pos = torch.tensor([0, 1, 2, 100, 4095, 8191, 20000, max_pos - 1])
    ang = oracle.rope_angles(pos, D, THETA)
    got = table[pos].cpu().double()
    err_c = (got[..., 0] - torch.cos(ang)).abs().max().item()
    err_s = (got[..., 1] - torch.sin(ang)).abs().max().item()
    say(f"table max abs err cos {err_c:.2e} sin {err_s:.2e}")
    assert err_c < 1e-7 and err_s < 1e-7  # fp32 rounding of the double values


def _run(pka, step, theta, max_pos):
    dev = torch.device("cuda")
    assert 0 <= int(step.positions.min()) and int(step.positions.max()) < max_pos  # table bounds, checked on the host
    qkv = W.fused_qkv(step)
    table = pka.rope_table(max_pos, step.head_dim, theta, dev)
    kc, vc = step.k_cache.to(dev), step.v_cache.to(dev)
    q_out = pka.fused_rope_kv_write(qkv.to(dev), step.positions.to(dev), step.slot_mapping.to(dev), table,
                                    step.num_q_heads, kc, vc)
    torch.cuda.synchronize()
    ref_q, ref_k, ref_v = oracle.fused_rope_kv_write(qkv, step.positions, step.slot_mapping, step.k_cache,
                                                     step.v_cache, step.num_q_heads, step.num_kv_heads, theta)
    return q_out, kc.cpu(), vc.cpu(), ref_q, ref_k, ref_v, qkv


def _check_step(pka, step, theta, max_pos):
    q_out, kc, vc, ref_q, ref_k, ref_v, qkv = _run(pka, step, theta, max_pos)
    # exact-rounded oracle values in fp64 for the ulp comparison
    rows = qkv.reshape(qkv.shape[0], step.num_q_heads + 2 * step.num_kv_heads, step.head_dim)
    q64 = oracle.rope(rows[:, :step.num_q_heads], step.positions, theta)
    k64 = oracle.rope(rows[:, step.num_q_heads:step.num_q_heads + step.num_kv_heads], step.positions, theta)
    check_rotated(q_out, q64, ref_q, f"{step.name} q")
    B = step.block_size
    live = step.slot_mapping >= 0
    slots = step.slot_mapping[live]
    blk, off = slots // B, slots % B
    check_rotated(kc[blk, off], k64[live], ref_k[blk, off], f"{step.name} k in the pool")
    assert torch.equal(vc[blk, off].view(torch.int16), rows[live, step.num_q_heads + step.num_kv_heads:].view(torch.int16))
    # untouched pool bytes (NaN payloads included) survive
    mask = torch.ones(kc.shape[:2], dtype=torch.bool)
    mask[blk, off] = False
    assert torch.equal(kc[mask].view(torch.int16), step.k_cache[mask].view(torch.int16))
    assert torch.equal(vc[mask].view(torch.int16), step.v_cache[mask].view(torch.int16))
    # and the written V matches the oracle's cache bit for bit
    assert torch.equal(vc.view(torch.int16), ref_v.view(torch.int16))


@pytest.mark.parametrize("seed", [0, 1])
def test_config5_rows(pka, seed):
    """The mixed step's 2,048 new rows (64 decodes + prefill chunks, positions
    up to ~7,700), bf16, 16 q / 8 kv heads, head_dim 128, NaN-poisoned pool."""
    step = W.config_5(seed=seed, poison=True)
    say(f"fused rope write, config 5 seed {seed}: {step.slot_mapping.numel()} rows, max pos {int(step.positions.max())}")
    _check_step(pka, step, THETA, 8192)


def test_fp16_small_heads_with_padding(pka):
    """fp16, 2 q / 2 kv heads, head_dim 64; some rows padded (slot -1), the
    first position 0 (identity) and the last one max_position - 1."""
    step = W.make_mixed_step(decode_ctx=[1, 64, 130], query_lens=[33, 17], cached_lens=[0, 80],
                             sharing=[False] * 5, dtype=torch.float16, num_q_heads=2, num_kv_heads=2, head_dim=64,
                             seed=41, poison=True)
    step.slot_mapping = step.slot_mapping.clone()
    step.slot_mapping[[1, 5, 20]] = -1
    step.positions = step.positions.clone()
    step.positions[-1] = 511
    say(f"fused rope write fp16 d64: {step.slot_mapping.numel()} rows, 3 padded")
    _check_step(pka, step, 1e4, 512)


def test_gqa_group_four_and_table_reuse(pka):
    """bf16, 32 q / 8 kv heads (group 4); one table serves two calls."""
    step = W.make_mixed_step(decode_ctx=[5, 300], query_lens=[64], cached_lens=[200], sharing=[False] * 3,
                             dtype=torch.bfloat16, num_q_heads=32, num_kv_heads=8, head_dim=128, seed=42,
                             poison=True)
    dev = torch.device("cuda")
    assert int(step.positions.max()) < 1024
    table = pka.rope_table(1024, 128, THETA, dev)
    qkv = W.fused_qkv(step).to(dev)
    outs = []
    for call in range(2):
        kc, vc = step.k_cache.to(dev), step.v_cache.to(dev)
        outs.append(pka.fused_rope_kv_write(qkv, step.positions.to(dev), step.slot_mapping.to(dev), table, 32, kc, vc))
    torch.cuda.synchronize()
    assert torch.equal(outs[0].cpu().view(torch.int16), outs[1].cpu().view(torch.int16))
    _check_step(pka, step, THETA, 1024)


def test_rotated_write_then_decode(pka):
    """End to end: rotated k written by the fused op, then paged decode over
    it, against the oracle's rotate-then-attend."""
    step = W.make_decode_step(context_lens=[40, 300, 1000], dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                              head_dim=128, seed=43, poison=True, write_new=True)
    dev = torch.device("cuda")
    assert int(step.positions.max()) < 2048
    table = pka.rope_table(2048, 128, THETA, dev)
    kc, vc = step.k_cache.to(dev), step.v_cache.to(dev)
    qkv = W.fused_qkv(step)
    q_rot = pka.fused_rope_kv_write(qkv.to(dev), step.positions.to(dev), step.slot_mapping.to(dev), table, 16, kc, vc)
    out = pka.paged_attn_decode_v1(q_rot, kc, vc, step.block_tables.to(dev), step.context_lens.to(dev), step.scale)
    torch.cuda.synchronize()
    ref_q, ref_k, ref_v = oracle.fused_rope_kv_write(qkv, step.positions, step.slot_mapping, step.k_cache,
                                                     step.v_cache, 16, 8, THETA)
    ref = oracle.decode(ref_q, ref_k, ref_v, step.block_tables, step.context_lens, step.scale)
    # q and k come from the GPU's own rounding of the rotation (within one unit
    # of the output spacing of the oracle's), so the decode sees inputs that
    # differ from the oracle's by up to one ulp: the looser of the two scaled
    # bounds (one input rounding per term) applies.
    assert_parity(out, ref, torch.bfloat16, "rotate-write-decode", weights_rounded=True)
