"""HIP-graph capture of the decode step (KV write + dispatched decode): every
replay, with eager work and synchronisations between replays, must reproduce
the eager result bit for bit (output and pool)."""

import pytest
import torch

import workloads as W
from tests.gpu_util import DevStep, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


@pytest.mark.parametrize("ctx", [[300, 1500, 77, 2000], [4000, 9000]], ids=["single-pass", "split-k"])
def test_graph_replay_matches_eager(pka, ctx):
    step = W.make_decode_step(context_lens=ctx, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8, head_dim=128,
                              seed=41, poison=True, write_new=True)
    ds = DevStep(step)
    S, Hq, D = step.q.shape
    max_ctx = step.max_context_len
    ws = torch.empty(max(1, pka.splitk_workspace_bytes(S, Hq, D, max_ctx)), dtype=torch.uint8, device="cuda")
    k0, v0 = ds.k_cache.clone(), ds.v_cache.clone()

    def run(out):
        pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
        pka.paged_attn_decode(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.context_lens, step.scale, max_ctx,
                              out=out, workspace=ws)

    say(f"graph capture of the decode step, ctx={ctx}")
    eager = torch.empty_like(ds.q)
    run(eager)
    torch.cuda.synchronize()
    pool_k, pool_v = ds.k_cache.clone(), ds.v_cache.clone()

    out = torch.empty_like(ds.q)
    ds.k_cache.copy_(k0)
    ds.v_cache.copy_(v0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(out)
    for rep in range(3):
        out.fill_(float("nan"))
        ds.k_cache.copy_(k0)
        ds.v_cache.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} output differs"
        assert torch.equal(ds.k_cache.view(torch.int16), pool_k.view(torch.int16)), f"replay {rep} K pool differs"
        assert torch.equal(ds.v_cache.view(torch.int16), pool_v.view(torch.int16)), f"replay {rep} V pool differs"
