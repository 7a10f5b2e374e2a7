"""Helpers for the GPU parity tests: move a seeded step to the device, run a
library call with the case printed first, compare against the oracle.

Two checks, both required:

1. The stated bound: max |gpu - oracle| <= 2e-3 (fp16 outputs) or 1.5e-2
   (bf16 outputs), no NaN or Inf.
2. A magnitude-scaled bound per element, so that a lost or extra key still
   fails when the outputs are small (a 16,384-token row has RMS ~0.013, and
   dropping a whole 256-token partition moves it by less than 1e-2):
       |gpu - ref| <= ulp_T(|ref|) + kappa * u_T * rms(ref over the head's D dims)
   where T is the output type, u_T its unit roundoff (2^-11 fp16, 2^-8 bf16)
   and ulp_T(x) the spacing of T at x.  The arithmetic fixes kappa:
   * decode, split-K and every path that rounds an fp32 result once: the
     rounding is at most half an ulp and the fp32 accumulation error stays a
     small fraction of the row's scale (kappa = 1/8);
   * prefill, whose softmax weights are rounded to T before the PV product:
     each weight carries a relative error of up to u_T, which moves an output
     by about u_T / sqrt(3) times the row's RMS per element (a random walk over
     the keys); kappa = 4 covers the largest of ~10^6 such elements.
"""

from __future__ import annotations

import sys

import torch

# Output tolerance (max abs error vs the fp64 oracle): fp16 2e-3, bf16 1.5e-2.
TOL = {torch.float16: 2e-3, torch.bfloat16: 1.5e-2}

# Unit roundoff and explicit mantissa bits of the output types.
UNIT_ROUNDOFF = {torch.float16: 2.0**-11, torch.bfloat16: 2.0**-8}
MANTISSA_BITS = {torch.float16: 10, torch.bfloat16: 7}
MIN_NORMAL_EXP = {torch.float16: -14, torch.bfloat16: -126}

KAPPA_SINGLE_ROUNDING = 0.125
KAPPA_WEIGHTS_ROUNDED = 4.0


def say(msg: str) -> None:
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


class DevStep:
    """Device copies of a workloads.PagedStep's tensors."""

    def __init__(self, step, device="cuda"):
        self.step = step
        d = device
        self.k_cache = step.k_cache.to(d)
        self.v_cache = step.v_cache.to(d)
        self.q = step.q.to(d)
        self.block_tables = step.block_tables.to(d)
        self.context_lens = step.context_lens.to(d)
        self.query_start_loc = step.query_start_loc.to(d)
        self.new_k = step.new_k.to(d) if step.new_k is not None else None
        self.new_v = step.new_v.to(d) if step.new_v is not None else None
        self.slot_mapping = step.slot_mapping.to(d) if step.slot_mapping is not None else None
        nd = step.num_decode
        self.decode_q = self.q[:nd]
        self.prefill_q = self.q[nd:]
        self.decode_block_tables = self.block_tables[:nd]
        self.prefill_block_tables = self.block_tables[nd:]
        self.decode_context_lens = self.context_lens[:nd]
        self.prefill_context_lens = self.context_lens[nd:]


def max_abs_err(gpu: torch.Tensor, ref: torch.Tensor) -> float:
    g = gpu.detach().to("cpu", torch.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert torch.isfinite(g).all(), "GPU output has NaN/Inf"
    return (g - ref).abs().max().item() if g.numel() else 0.0


def ulp(ref: torch.Tensor, dtype: torch.dtype) -> torch.Tensor:
    """Spacing of `dtype` at |ref| (float64 in, float64 out); below the
    smallest normal the subnormal spacing."""
    a = ref.abs()
    exp = torch.floor(torch.log2(torch.where(a > 0, a, torch.ones_like(a))))
    exp = torch.where(a > 0, exp, torch.full_like(a, float(MIN_NORMAL_EXP[dtype])))
    exp = torch.clamp(exp, min=MIN_NORMAL_EXP[dtype])
    return torch.pow(2.0, exp - MANTISSA_BITS[dtype])


def scaled_bound(ref: torch.Tensor, dtype: torch.dtype, weights_rounded: bool = False) -> torch.Tensor:
    """Per-element bound of the magnitude-scaled check (see the module text)."""
    ref = ref.to(torch.float64)
    rms = ref.pow(2).mean(dim=-1, keepdim=True).sqrt()
    kappa = KAPPA_WEIGHTS_ROUNDED if weights_rounded else KAPPA_SINGLE_ROUNDING
    return ulp(ref, dtype) + kappa * UNIT_ROUNDOFF[dtype] * rms


def scaled_violation(out: torch.Tensor, ref: torch.Tensor, dtype: torch.dtype, weights_rounded: bool = False):
    """(worst err / bound ratio, number of elements above their bound, index of
    the worst element) of `out` against `ref` (both compared in float64)."""
    o = out.detach().to("cpu", torch.float64)
    ref = ref.to(torch.float64)
    assert o.shape == ref.shape, (o.shape, ref.shape)
    if o.numel() == 0:
        return 0.0, 0, None
    ratio = (o - ref).abs() / scaled_bound(ref, dtype, weights_rounded)
    ratio = torch.where(torch.isfinite(ratio), ratio, torch.full_like(ratio, float("inf")))
    worst = int(torch.argmax(ratio))
    idx = tuple(int(i) for i in torch.unravel_index(torch.tensor(worst), ratio.shape))
    return ratio.flatten()[worst].item(), int((ratio > 1.0).sum()), idx


def assert_parity(gpu: torch.Tensor, ref: torch.Tensor, dtype: torch.dtype, what: str,
                  weights_rounded: bool = False) -> float:
    """Both checks: the stated max-abs tolerance and the magnitude-scaled
    bound (weights_rounded=True for the prefill kernel's outputs)."""
    err = max_abs_err(gpu, ref)
    tol = TOL[dtype]
    worst, nbad, idx = scaled_violation(gpu, ref, dtype, weights_rounded)
    say(f"{what}: max abs err {err:.3e} (tol {tol:.1e}); scaled check worst {worst:.3f} of its bound at {idx}")
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
    assert nbad == 0, f"{what}: {nbad} elements above the magnitude-scaled bound (worst {worst:.2f}x at {idx})"
    return err
