"""HIP-graph capture of the decode step (KV write + dispatched decode, as two
launches and with the write folded into the decode launch) and of the mixed
step (fused rotary write, decode, split prefill): every replay, with eager
work and synchronisations between replays, is checked against the oracle -
output within the parity bounds, pools bit-exact where the write is a byte
copy - and must reproduce the eager launch bit for bit."""

import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import DevStep, assert_parity, say

pytestmark = pytest.mark.gpu

ROPE_THETA = 1e6


@pytest.fixture(scope="module")
def pka():
    import paged_kv_attention_21_amd as pka

    return pka


def bits(t):
    return t.detach().cpu().view(torch.int16)


@pytest.mark.parametrize("fused", [False, True], ids=["write+decode", "decode_append"])
@pytest.mark.parametrize("ctx", [[300, 1500, 77, 2000], [4000, 9000]], ids=["single-pass", "split-k"])
@pytest.mark.parametrize("hq", [16, 64], ids=["group2", "group8"])
def test_graph_replay_matches_oracle(pka, ctx, fused, hq):
    """Groups of two run on the vector path, groups of eight on the matrix
    cores; both are captured and replayed."""
    step = W.make_decode_step(context_lens=ctx, dtype=torch.bfloat16, num_q_heads=hq, num_kv_heads=8, head_dim=128,
                              seed=41, poison=True, write_new=True)
    ds = DevStep(step)
    S, Hq, D = step.q.shape
    max_ctx = step.max_context_len
    ws = pka.splitk_workspace(S, Hq, D, max_ctx, "cuda")
    k0, v0 = ds.k_cache.clone(), ds.v_cache.clone()

    ref_k, ref_v = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, step.k_cache, step.v_cache)
    ref = oracle.decode(step.q, ref_k, ref_v, step.block_tables, step.context_lens, step.scale)

    def run(out):
        if fused:
            pka.paged_attn_decode_append(ds.q, ds.new_k, ds.new_v, ds.k_cache, ds.v_cache, ds.block_tables,
                                         ds.context_lens, step.scale, max_ctx, out=out, workspace=ws)
            return
        pka.kv_cache_write(ds.new_k, ds.new_v, ds.slot_mapping, ds.k_cache, ds.v_cache)
        pka.paged_attn_decode(ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ds.context_lens, step.scale, max_ctx,
                              out=out, workspace=ws)

    say(f"graph capture of the decode step, ctx={ctx}, fused={fused}, Hq={hq}, "
        f"variant={pka.decode_choose_variant(S, step.num_kv_heads, max_ctx)}")
    eager = torch.empty_like(ds.q)
    run(eager)
    torch.cuda.synchronize()
    assert_parity(eager, ref, step.dtype, "eager decode step")
    assert torch.equal(bits(ds.k_cache), ref_k.view(torch.int16)), "eager K pool differs from the oracle's"
    assert torch.equal(bits(ds.v_cache), ref_v.view(torch.int16)), "eager V pool differs from the oracle's"

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
        assert_parity(out, ref, step.dtype, f"graph replay {rep}")
        assert torch.equal(bits(ds.k_cache), ref_k.view(torch.int16)), f"replay {rep} K pool differs from the oracle's"
        assert torch.equal(bits(ds.v_cache), ref_v.view(torch.int16)), f"replay {rep} V pool differs from the oracle's"
        assert torch.equal(bits(out), bits(eager)), f"replay {rep} output differs from the eager launch"


@pytest.mark.parametrize("two_streams", [False, True], ids=["one-stream", "decode-on-side-stream"])
def test_mixed_step_graph_replay_matches_oracle(pka, two_streams):
    """The mixed step as the benchmark replays it: fused rotary + KV write of
    the new rows, decode rows, and prefill chunks whose long prefix is split,
    captured once and replayed three times.  The oracle rotates with its own
    fp64 arithmetic, so its pool and q differ from the GPU's rounding by at most
    one unit of the output spacing in the rotated k and q (V is a byte copy and
    must match bit for bit); the attention rows are checked with the bound for
    one input rounding per term."""
    step = W.make_mixed_step(decode_ctx=[40, 1300, 17, 700], query_lens=[37, 200, 64], cached_lens=[0, 2900, 128],
                             sharing=[False] * 7, dtype=torch.bfloat16, num_q_heads=16, num_kv_heads=8,
                             head_dim=128, seed=43, poison=True)
    ds = DevStep(step)
    nd = step.num_decode
    S, Hq, D = step.q.shape
    Hkv = step.num_kv_heads
    max_dec = int(step.decode_context_lens.max())
    mcl = int(step.prefill_context_lens.max())
    ws = pka.splitk_workspace(nd, Hq, D, max_dec, "cuda")
    pws = pka.prefill_workspace(step.num_prefill, step.num_prefill_rows, Hq, Hkv, D, mcl, "cuda")
    assert pka.prefill_workspace_bytes(step.num_prefill, step.num_prefill_rows, Hq, Hkv, D, mcl) > 0
    table = pka.rope_table(4096, D, ROPE_THETA, "cuda")
    qkv_host = W.fused_qkv(step)
    qkv = qkv_host.cuda()
    pos = step.positions.cuda()
    k0, v0 = ds.k_cache.clone(), ds.v_cache.clone()
    q_rot = torch.empty_like(ds.q)

    rq, rk, rv = oracle.fused_rope_kv_write(qkv_host, step.positions, step.slot_mapping, step.k_cache, step.v_cache,
                                            Hq, Hkv, ROPE_THETA)
    ref_dec = oracle.decode(rq[:nd], rk, rv, step.decode_block_tables, step.decode_context_lens, step.scale)
    ref_pre = oracle.prefill(rq[nd:], rk, rv, step.prefill_block_tables, step.prefill_context_lens,
                             step.query_start_loc, step.scale)
    written = step.slot_mapping[step.slot_mapping >= 0]
    untouched = torch.ones(step.k_cache.shape[:2], dtype=torch.bool)
    untouched[written // step.block_size, written % step.block_size] = False

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

    def check(out, what):
        assert_parity(out[:nd], ref_dec, step.dtype, f"{what} decode rows", weights_rounded=True)
        assert_parity(out[nd:], ref_pre, step.dtype, f"{what} prefill rows", weights_rounded=True)
        kb, vb = bits(ds.k_cache), bits(ds.v_cache)
        assert torch.equal(vb, rv.view(torch.int16)), f"{what}: V pool differs from the oracle's"
        assert torch.equal(kb[untouched], rk.view(torch.int16)[untouched]), f"{what}: K bytes outside the slots changed"
        got = kb[~untouched].view(torch.bfloat16).double()
        want = rk[~untouched].double()
        assert (got - want).abs().max().item() <= 2.0**-7 * want.abs().max().item(), f"{what}: rotated K off by > 1 ulp"

    say(f"graph capture of the mixed step, two streams: {two_streams}")
    eager = torch.empty_like(ds.q)
    run(eager)
    torch.cuda.synchronize()
    check(eager, "eager mixed step")
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
        check(out, f"graph replay {rep}")
        assert torch.equal(bits(out), bits(eager)), f"replay {rep} output differs from the eager launch"
