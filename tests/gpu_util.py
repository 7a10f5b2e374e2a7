"""Helpers for the GPU parity tests: move a seeded step to the device, run a
library call with the case printed first, compare against the oracle."""

from __future__ import annotations

import sys

import torch

# Output tolerance (max abs error vs the fp64 oracle): fp16 2e-3, bf16 1.5e-2.
TOL = {torch.float16: 2e-3, torch.bfloat16: 1.5e-2}


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


def assert_parity(gpu: torch.Tensor, ref: torch.Tensor, dtype: torch.dtype, what: str) -> float:
    err = max_abs_err(gpu, ref)
    tol = TOL[dtype]
    say(f"{what}: max abs err {err:.3e} (tol {tol:.1e})")
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"
    return err
