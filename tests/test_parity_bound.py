"""The parity checks must be able to fail at full size.

At the long-context sizes the outputs are small (config 4: RMS ~0.013, max
~0.056), so the stated max-abs tolerance alone (1.5e-2 for bf16) would accept
a kernel that loses a whole 256-token partition.  The magnitude-scaled bound
in tests/gpu_util.py is checked here, on the CPU, against the oracle's own
results:

* it accepts the correctly rounded oracle result (decode) and the oracle
  recomputed with the softmax weights rounded to bf16, as the prefill kernel
  does (prefill);
* it rejects plausible kernel mistakes built from the oracle's own functions -
  a dropped split-K partition and a dropped last KV block at config-4 size, and
  a causal mask shifted by one key in the long chunk of the config-5 step -
  including the ones the stated tolerance alone lets through.
"""

import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import TOL, say, scaled_violation

BF16 = torch.bfloat16


def rounded(x: torch.Tensor, dtype) -> torch.Tensor:
    """Round a float64 result to the output type (nearest even), back in float64."""
    return x.to(dtype).to(torch.float64)


def stated_ok(out, ref, dtype) -> bool:
    return (out - ref).abs().max().item() <= TOL[dtype]


@pytest.fixture(scope="module")
def cfg4():
    step = W.config_4(seed=0, poison=False)
    ref = oracle.decode(step.decode_q, step.k_cache, step.v_cache, step.decode_block_tables,
                        step.decode_context_lens, step.scale)
    return step, ref


def test_config4_bound_accepts_rounded_oracle(cfg4):
    step, ref = cfg4
    worst, nbad, _ = scaled_violation(rounded(ref, BF16), ref, BF16)
    say(f"config 4, oracle rounded to bf16: worst {worst:.3f} of the bound")
    assert nbad == 0 and worst <= 1.0


def test_config4_dropped_partition_rejected(cfg4):
    """Merge every (sequence, head) without its partition 37 (of 64)."""
    step, ref = cfg4
    m, l, po, npart = oracle.decode_partitions(step.decode_q, step.k_cache, step.v_cache, step.decode_block_tables,
                                               step.decode_context_lens, step.scale, 256)
    keep = [p for p in range(int(npart.max())) if p != 37]
    mutant = oracle.merge_partitions(m[:, :, keep], l[:, :, keep], po[:, :, keep], npart - 1)
    out = rounded(mutant, BF16)
    err = (out - ref).abs().max().item()
    worst, nbad, _ = scaled_violation(out, ref, BF16)
    say(f"dropped partition: max abs err {err:.2e} (stated bound passes: {stated_ok(out, ref, BF16)}); "
        f"scaled check: {nbad} elements over, worst {worst:.1f}x")
    assert stated_ok(out, ref, BF16), "expected the stated tolerance alone to miss this mistake"
    assert nbad > 0


def test_config4_dropped_last_block_rejected(cfg4):
    """Every sequence decoded without its last 16-token block."""
    step, ref = cfg4
    short = step.decode_context_lens - step.block_size
    mutant = oracle.decode(step.decode_q, step.k_cache, step.v_cache, step.decode_block_tables, short, step.scale)
    out = rounded(mutant, BF16)
    err = (out - ref).abs().max().item()
    worst, nbad, _ = scaled_violation(out, ref, BF16)
    say(f"dropped last block: max abs err {err:.2e} (stated bound passes: {stated_ok(out, ref, BF16)}); "
        f"scaled check: {nbad} elements over, worst {worst:.1f}x")
    assert stated_ok(out, ref, BF16), "expected the stated tolerance alone to miss this mistake"
    assert nbad > 0


def _long_chunk(step):
    """Index, packed row range and cached length of the prefill chunk with the
    longest cached prefix."""
    qsl = step.query_start_loc
    cached = step.prefill_context_lens - (qsl[1:] - qsl[:-1])
    j = int(torch.argmax(cached))
    return j, int(qsl[j]), int(qsl[j + 1]), int(cached[j])


def _rows_with_keys(step, j, start, end, cached, keys_of_row, weights_dtype=None):
    """Float64 outputs of chunk j's rows where row i sees keys_of_row(i)
    keys, built from the oracle's materialisation; with weights_dtype the
    softmax weights are rounded to that type before the PV product."""
    Hq, Hkv = step.num_q_heads, step.num_kv_heads
    ctx = int(step.prefill_context_lens[j])
    K = oracle.materialize(step.k_cache, step.prefill_block_tables[j], ctx)
    V = oracle.materialize(step.v_cache, step.prefill_block_tables[j], ctx)
    out = torch.empty((end - start, Hq, step.head_dim), dtype=torch.float64)
    for i in range(end - start):
        n = keys_of_row(i)
        qi = oracle.widen(step.prefill_q[start + i])
        for h in range(Hq):
            g = oracle.kv_head_of(h, Hq, Hkv)
            if weights_dtype is None:
                out[i, h] = oracle.attend(qi[h], K[:n, g], V[:n, g], step.scale)
            else:
                s = step.scale * (K[:n, g] @ qi[h])
                w = torch.exp(s - s.max()).to(weights_dtype).to(torch.float64)
                out[i, h] = (w @ V[:n, g]) / w.sum()
    return out


@pytest.fixture(scope="module")
def cfg5():
    step = W.config_5(seed=0, poison=False)
    ref = oracle.prefill(step.prefill_q, step.k_cache, step.v_cache, step.prefill_block_tables,
                         step.prefill_context_lens, step.query_start_loc, step.scale)
    return step, ref


def test_config5_bound_accepts_weights_rounded_like_the_kernel(cfg5):
    """The prefill kernel rounds each softmax weight to bf16 before PV; the
    oracle recomputed that way (then rounded to bf16) must pass the prefill
    bound on the long chunk's rows."""
    step, ref = cfg5
    j, start, end, cached = _long_chunk(step)
    sim = _rows_with_keys(step, j, start, end, cached, lambda i: oracle.visible_keys(cached, i), weights_dtype=BF16)
    worst, nbad, _ = scaled_violation(rounded(sim, BF16), ref[start:end], BF16, weights_rounded=True)
    say(f"config 5 long chunk with bf16 weights: worst {worst:.3f} of the prefill bound")
    assert nbad == 0


@pytest.mark.parametrize("shift", [-1, 1], ids=["one-key-fewer", "one-key-more"])
def test_config5_causal_shift_rejected(cfg5, shift):
    """The long chunk's rows (after a 2,560-token prefix) each see one key
    fewer or one more than the bottom-right mask allows (the last row keeps its
    keys when shifted up: there is no later key)."""
    step, ref = cfg5
    j, start, end, cached = _long_chunk(step)
    assert cached >= 512
    qlen = end - start
    mutant = ref.clone()
    mutant[start:end] = _rows_with_keys(
        step, j, start, end, cached,
        lambda i: min(oracle.visible_keys(cached, i) + shift, cached + qlen))
    out = rounded(mutant, BF16)
    err = (out - ref).abs().max().item()
    worst, nbad, _ = scaled_violation(out, ref, BF16, weights_rounded=True)
    say(f"causal shift {shift:+d}: max abs err {err:.2e} (stated bound passes: {stated_ok(out, ref, BF16)}); "
        f"scaled check: {nbad} elements over, worst {worst:.1f}x")
    assert nbad > 0


def test_ulp_spacing_matches_the_types():
    """ulp() is the spacing of the type: x + ulp(x) is the next representable value."""
    from tests.gpu_util import ulp

    for dtype in (torch.float16, BF16):
        x = torch.tensor([1.0, 0.013, 0.056, 3.5, 1e-5, 0.0], dtype=torch.float64)
        u = ulp(x, dtype)
        xs = x.to(dtype).to(torch.float64)
        up = (xs + u).to(dtype).to(torch.float64)
        half = (xs + 0.49 * u).to(dtype).to(torch.float64)
        assert torch.all(up > xs) and torch.equal(half, xs), dtype
