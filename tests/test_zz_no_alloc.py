"""The allocation-free decode entry point (pka_paged_attn_decode_noalloc),
called through the C ABI: its output must equal pka_paged_attn_decode's (the
same kernels, so bit for bit) and the oracle's within the parity bounds, on
two calls in a row - the second with a smaller input, so the library's
scratch holds the first call's partition states when it starts - on the
split-K path and on the single pass.  Requests beyond the scratch are refused
before any launch."""

import ctypes

import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DevStep, assert_parity, say

pytestmark = pytest.mark.gpu

PKA_ERR_SCRATCH = 7
SCRATCH_BYTES = 32 * 1024 * 1024


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


def _noalloc_c_abi(pka, ds, max_ctx, out):
    """pka_paged_attn_decode_noalloc through ctypes, arguments marshalled here."""
    lib = pka._lib.lib
    S, Hq, _ = ds.decode_q.shape
    st = lib.pka_paged_attn_decode_noalloc(
        ctypes.c_void_p(ds.decode_q.data_ptr()), ctypes.c_void_p(ds.k_cache.data_ptr()),
        ctypes.c_void_p(ds.v_cache.data_ptr()), ctypes.c_void_p(ds.decode_block_tables.data_ptr()),
        ctypes.c_void_p(ds.decode_context_lens.data_ptr()), S, Hq, ds.decode_block_tables.shape[1], int(max_ctx),
        float(ds.step.scale), ctypes.c_void_p(out.data_ptr()), pka.cache_desc(ds.k_cache),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st


def _check_case(pka, step, what):
    ds = DevStep(step)
    k_ref, v_ref = step.k_cache, step.v_cache
    if step.new_k is not None:
        # The step's new rows go in first (their slots hold NaN until then).
        pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
        k_ref, v_ref = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, k_ref, v_ref)
    S, Hq, D = step.decode_q.shape
    max_ctx = int(step.decode_context_lens.max())
    variant = pka.decode_choose_variant(S, step.num_kv_heads, max_ctx)
    say(f"noalloc {what}: S={S} max_ctx={max_ctx} variant={variant}")
    out = torch.full_like(ds.decode_q, float("nan"))
    assert _noalloc_c_abi(pka, ds, max_ctx, out) == 0
    ref_out = pka.paged_attn_decode(ds.decode_q, ds.k_cache, ds.v_cache, ds.decode_block_tables,
                                    ds.decode_context_lens, step.scale, max_ctx,
                                    workspace=pka.splitk_workspace(S, Hq, D, max_ctx, "cuda"))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), ref_out.cpu().view(torch.int16)), \
        f"{what}: differs from pka_paged_attn_decode"
    ref = oracle.decode(step.decode_q, k_ref, v_ref, step.decode_block_tables, step.decode_context_lens, step.scale)
    assert_parity(out, ref, step.dtype, f"noalloc {what}")
    return variant


def test_noalloc_split_then_smaller(pka):
    """Split-K twice in a row: config 4 (4 x 16,384 tokens), then a smaller
    batch of shorter, ragged contexts."""
    assert _check_case(pka, W.config_4(seed=0, poison=True), "config 4") == 2
    step = W.make_decode_step(context_lens=[3000, 300, 7777], dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                              head_dim=128, seed=51, poison=True)
    assert _check_case(pka, step, "smaller split-K batch") == 2


def test_noalloc_single_pass_then_smaller(pka):
    """The single pass (no scratch): config 3 (256 sequences), then a smaller batch."""
    assert _check_case(pka, W.config_3(seed=0, poison=True), "config 3") == 1
    g = torch.Generator().manual_seed(52)
    ctx = torch.randint(100, 2049, (80,), generator=g).tolist()
    step = W.make_decode_step(context_lens=ctx, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8, head_dim=128,
                              seed=52, poison=True)
    assert _check_case(pka, step, "smaller single-pass batch") == 1


def test_noalloc_group8_split_then_single(pka):
    """Groups of eight (the matrix-core path): a split-K batch, then a
    single-pass batch, both through the scratch-free entry point."""
    step = W.make_decode_step(context_lens=[9000, 40, 5000], dtype=torch.bfloat16, num_q_heads=64, num_kv_heads=8,
                              head_dim=128, seed=53, poison=True)
    assert _check_case(pka, step, "group-8 split-K batch") == 2
    g = torch.Generator().manual_seed(54)
    ctx = torch.randint(100, 2049, (300,), generator=g).tolist()
    step = W.make_decode_step(context_lens=ctx, dtype=torch.bfloat16, num_q_heads=64, num_kv_heads=8, head_dim=128,
                              seed=54, poison=True)
    assert _check_case(pka, step, "group-8 single-pass batch") == 1


def test_noalloc_refuses_beyond_scratch(pka):
    """A split-K request whose partition states exceed the built-in scratch is
    refused with PKA_ERR_SCRATCH before anything is launched (the pointers are
    never dereferenced: sizes are checked first)."""
    lib = pka._lib.lib
    S, Hq, D, ctx = 4, 16, 128, 300_000
    assert pka.splitk_workspace_bytes(S, Hq, D, ctx) > SCRATCH_BYTES
    desc = pka._lib.CacheDesc(4700, 16, 8, D, 1)
    dummy = torch.empty(16, dtype=torch.bfloat16, device="cuda")
    p = ctypes.c_void_p(dummy.data_ptr())
    st = lib.pka_paged_attn_decode_noalloc(p, p, p, p, p, S, Hq, 20000, ctx, 0.088, p, desc, None)
    assert st == PKA_ERR_SCRATCH, st
    assert "scratch" in lib.pka_status_str(st).decode()
