"""HIP-graph capture of the decode step (KV write + dispatched decode, as two
launches and with the write folded into the decode launch) and of
the mixed step (fused rotary write, decode, split prefill + merge): every
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


@pytest.mark.parametrize("fused", [False, True], ids=["write+decode", "decode_append"])
@pytest.mark.parametrize("ctx", [[300, 1500, 77, 2000], [4000, 9000]], ids=["single-pass", "split-k"])
def test_graph_replay_matches_eager(pka, ctx, fused):
    step = W.make_decode_step(context_lens=ctx, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8, head_dim=128,
                              seed=41, poison=True, write_new=True)
    ds = DevStep(step)
    S, Hq, D = step.q.shape
    max_ctx = step.max_context_len
    ws = torch.empty(max(1, pka.splitk_workspace_bytes(S, Hq, D, max_ctx)), dtype=torch.uint8, device="cuda")
    k0, v0 = ds.k_cache.clone(), ds.v_cache.clone()

    def run(out):
        if fused:
            pka.paged_attn_decode_append(ds.q, ds.new_k, ds.new_v, ds.k_cache, ds.v_cache, ds.block_tables,
                                         ds.context_lens, step.scale, max_ctx, out=out, workspace=ws)
            return
        pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
        pka.paged_attn_decode(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.context_lens, step.scale, max_ctx,
                              out=out, workspace=ws)

    say(f"graph capture of the decode step, ctx={ctx}, fused={fused}")
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


@pytest.mark.parametrize("two_streams", [False, True], ids=["one-stream", "decode-on-side-stream"])
def test_mixed_step_graph_replay_matches_eager(pka, two_streams):
    """The mixed step as the benchmark replays it: fused rotary + KV write of
    the new rows, decode rows, and prefill chunks whose long prefix is split
    (attention + merge kernels), captured once and replayed three times."""
    step = W.make_mixed_step(decode_ctx=[40, 1300, 17, 700], query_lens=[37, 200, 64], cached_lens=[0, 2900, 128],
                             sharing=[False] * 7, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                             head_dim=128, seed=43, poison=True)
    ds = DevStep(step)
    nd = step.num_decode
    S, Hq, D = step.q.shape
    max_dec = int(step.decode_context_lens.max())
    mcl = int(step.prefill_context_lens.max())
    ws = torch.empty(max(1, pka.splitk_workspace_bytes(nd, Hq, D, max_dec)), dtype=torch.uint8, device="cuda")
    pws = torch.empty(max(1, pka.prefill_workspace_bytes(step.num_prefill, step.num_prefill_rows, Hq,
                                                         step.num_kv_heads, D, mcl)), dtype=torch.uint8,
                      device="cuda")
    assert pka.prefill_workspace_bytes(step.num_prefill, step.num_prefill_rows, Hq, step.num_kv_heads, D, mcl) > 0
    table = pka.rope_table(4096, D, 1e6, "cuda")
    qkv = W.fused_qkv(step).cuda()
    pos = step.positions.cuda()
    k0, v0 = ds.k_cache.clone(), ds.v_cache.clone()
    q_rot = torch.empty_like(ds.q)

    side = torch.cuda.Stream()  # default priority

    def run(out):
        pka.fused_rope_kv_write(qkv, pos, ds.slot_mapping, table, Hq, ds.k_cache, ds.v_cache, q_out=q_rot)
        if two_streams:
            # Fork: the decode rows on a side stream beside the prefill; join before the end.
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                pka.paged_attn_decode(q_rot[:nd], ds.k_cache, ds.v_cache, ds.block_tables[:nd], ds.context_lens[:nd],
                                      step.scale, max_dec, out=out[:nd], workspace=ws)
        else:
            pka.paged_attn_decode(q_rot[:nd], ds.k_cache, ds.v_cache, ds.block_tables[:nd], ds.context_lens[:nd],
                                  step.scale, max_dec, out=out[:nd], workspace=ws)
        pka.paged_attn_prefill(q_rot[nd:], ds.k_cache, ds.v_cache, ds.block_tables[nd:], ds.context_lens[nd:],
                               ds.query_start_loc, step.scale, step.max_query_len, mcl, out=out[nd:], workspace=pws)
        if two_streams:
            torch.cuda.current_stream().wait_stream(side)

    say(f"graph capture of the mixed step, two streams: {two_streams}")
    eager = torch.empty_like(ds.q)
    run(eager)
    torch.cuda.synchronize()
    assert torch.isfinite(eager.float()).all()
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
        pws.fill_(0xFF)  # stale split states must not matter
        ds.k_cache.copy_(k0)
        ds.v_cache.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"replay {rep}")
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep} output differs"
        assert torch.equal(ds.k_cache.view(torch.int16), pool_k.view(torch.int16)), f"replay {rep} K pool differs"
        assert torch.equal(ds.v_cache.view(torch.int16), pool_v.view(torch.int16)), f"replay {rep} V pool differs"
