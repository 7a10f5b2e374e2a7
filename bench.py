#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Default workload (the one the headline metric is quoted on): one decode step
of a Qwen3-0.6B-shaped attention layer - bf16, 16 query / 8 KV heads, head
dim 128, KV block 16, 256 sequences with context uniform in [100, 2048] -
i.e. the KV-cache write of the 256 new rows followed by the dispatched paged
decode that reads them.  A "step" is that write plus that decode.

Prints ONE JSON line: `value` is the step's algorithmic HBM bytes (decode
K/V/q/out/tables + write rows) divided by the measured step time, in GB/s;
`roofline` reports the decode kernel alone (algorithmic bytes per launch over
its average launch time, from HIP events on the launch stream) against the
8 TB/s HBM peak; `cpu_baseline` times the fp64 CPU oracle on the same inputs.

Other workloads (--workload): `splitk` (4 x 16,384-token split-K decode),
`mixed` (KV write + decode + ragged causal prefill in one step),
`sweep` (single-request fp16 decode at 128 / 1,024 / 4,096 tokens, next to a
materialise-then-attend arm), `single` (the 128-token request alone),
`prefill_long` (4 x 2,048 causal rows after 6,144 cached tokens), `shapes`
(the decode batch at other head / group / block shapes), `prefill_shapes`
(the long prefill's chunks at other head / group / block shapes),
`rope_kv_write`, `block_manager`, `copy` (a device copy, for counter
calibration).

Inputs are seeded synthetic tensors already resident in HBM when timing
starts.  Pools are rotated over several device copies so no step reads what
the previous one left in the 256 MiB Infinity Cache.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 MFMA, published
ROTATE_BYTES = 1 << 30          # rotate pools until at least 1 GiB is cycled
ROPE_THETA = 1e6               # rotary base of the rope_kv_write workload (Qwen3 checkpoints)

# HBM bytes per launch of each workload's dominant kernel, from rocprofv3
# FETCH_SIZE (x 2.0, the factor a 1 GiB copy calibrates) + WRITE_SIZE runs
# (profiles/traffic_fetch_write.md), valid only for the kernel source they were
# taken on: (source file, sha256 prefix, bytes).  The bench line names the
# source of its traffic figure, or why it is null.
TRAFFIC_PROFILE = "profiles/traffic_fetch_write.md"
RECORDED_TRAFFIC = {
    "decode_step": ("decode_impl.h", "508287ea44944b78", 1191837382),
    "splitk": ("decode_impl.h", "508287ea44944b78", 269528776),
    "mixed": ("prefill.hip", "0f354d6425638b9e", 50251018),
    "prefill_long": ("prefill.hip", "0f354d6425638b9e", 465589472),
    "rope_kv_write": ("rope_kv.hip", "6db5d8adbcf54e98", 34923040),
}


def recorded_traffic(workload):
    """(traffic bytes or None, a note on where the figure comes from): the
    recorded counters if the dominant kernel's source is unchanged since they
    were taken, else None."""
    import hashlib

    if workload not in RECORDED_TRAFFIC:
        return None, "no counter run recorded for this workload"
    fname, digest, nbytes = RECORDED_TRAFFIC[workload]
    path = os.path.join(ROOT, "paged_kv_attention_21_amd", "csrc", fname)
    with open(path, "rb") as f:
        now = hashlib.sha256(f.read()).hexdigest()[:16]
    if now != digest:
        return None, (f"counters were taken on csrc/{fname} sha256 {digest}, the source is now {now}: "
                      "not measured for this source")
    return nbytes, (f"recorded, not measured in this run: rocprofv3 FETCH_SIZE x 2.0 + WRITE_SIZE per dispatch "
                    f"({TRAFFIC_PROFILE}), kernel source csrc/{fname} sha256 {digest} (unchanged)")


def parse_args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode_step",
                   choices=["decode_step", "splitk", "mixed", "sweep", "single", "copy", "rope_kv_write",
                            "block_manager", "prefill_long", "shapes", "prefill_shapes"])
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--settle-ms", type=float, default=500.0,
                   help="untimed stepping before the first timed block (clock/power ramp), once per process")
    p.add_argument("--rotate", type=int, default=0, help="pool copies to cycle (0 = enough for 1 GiB)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-arms", action="store_true",
                   help="skip the comparison arms (unified prefill, eager rotary) - for profiling the kernels alone")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-graph", action="store_true", help="time eager launches only (no HIP-graph replay)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def fingerprint():
    prop = torch.cuda.get_device_properties(0)
    return {
        "name": prop.name,
        "arch": getattr(prop, "gcnArchName", ""),
        "cus": prop.multi_processor_count,
        "hbm_gib": round(prop.total_memory / 2**30, 1),
        "torch": torch.__version__,
        "hip": torch.version.hip,
    }


class Pools:
    """R device copies of a step's KV pool (tables, q and new rows shared)."""

    def __init__(self, step, rotate):
        dev = torch.device("cuda:0")
        pool_bytes = 2 * step.k_cache.numel() * step.k_cache.element_size()
        self.R = rotate or max(2, math.ceil(ROTATE_BYTES / pool_bytes))
        k = step.k_cache.to(dev)
        v = step.v_cache.to(dev)
        self.k = [k] + [k.clone() for _ in range(self.R - 1)]
        self.v = [v] + [v.clone() for _ in range(self.R - 1)]
        self.q = step.q.to(dev)
        self.bt = step.block_tables.to(dev)
        self.cl = step.context_lens.to(dev)
        self.qsl = step.query_start_loc.to(dev)
        self.new_k = step.new_k.to(dev) if step.new_k is not None else None
        self.new_v = step.new_v.to(dev) if step.new_v is not None else None
        self.slots = step.slot_mapping.to(dev) if step.slot_mapping is not None else None
        self.out = torch.empty_like(self.q)


def percentiles(xs, qs=(10, 50, 90)):
    """Nearest-rank percentiles of a list of timings."""
    xs = sorted(xs)
    return [xs[min(len(xs) - 1, max(0, math.ceil(q / 100 * len(xs)) - 1))] for q in qs]


# Untimed stepping once per process before the first timed block: on MI355X
# the first ~0.1-0.3 s of sustained load run a few percent slower (clock and
# power ramp), which would otherwise penalise whichever arm is timed first.
SETTLE_S = 0.5
_settled = False


def settle(run_once):
    """Keep the GPU busy with untimed steps for SETTLE_S seconds, once per process."""
    global _settled
    if _settled:
        return
    _settled = True
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(8):
            run_once(i)
            i += 1
        torch.cuda.synchronize()


def timed_loop(launch, n_phases, steps, warmup, stats=None):
    """Run `launch(i, ev)` warmup + steps times; `ev` is a list of n_phases+1
    events the launcher records between its kernels.  Returns (wall ms per
    step, per-phase mean ms from events); with `stats` (a dict), also stores
    each phase's p10 / p50 / p90 in ms under stats["pct"]."""
    for i in range(warmup):
        launch(i, None)
    settle(lambda i: launch(warmup + i, None))
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_phases + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        launch(warmup + i, evs[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = [[e[p].elapsed_time(e[p + 1]) for e in evs] for p in range(n_phases)]
    if stats is not None:
        stats["pct"] = [percentiles(x) for x in per]
    return wall_ms, [sum(x) / steps for x in per]


SWEEP_BATCH = 100  # calls per captured batch in the single-request sweep


def graph_batch_us(fn, batch, replays, warmup):
    """Capture `fn` (a batch of `batch` back-to-back calls) as one HIP graph,
    replay it, and return the p10 / p50 / p90 over replays of the device time
    per call in microseconds (events on the replay stream / batch)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(warmup):
        g.replay()
    settle(lambda i: g.replay())
    torch.cuda.synchronize()
    per = []
    for _ in range(replays):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        b.synchronize()
        per.append(a.elapsed_time(b) * 1e3 / batch)
    return percentiles(per)


KERNEL_BATCH = 20  # back-to-back calls per replay when timing a kernel for its roofline figure


def back_to_back_us(call, R, warmup):
    """Device time per call of call(r) (r = pool copy), from replays of one
    HIP graph of KERNEL_BATCH back-to-back calls over the rotated pools: p10 /
    p50 / p90 in microseconds.  The host launch path drops out, so the figure
    is the kernels' time plus the gaps between dependent launches - what a
    profiler's kernel trace averages."""
    def fn():
        for i in range(KERNEL_BATCH):
            call(i % R)
    return graph_batch_us(fn, KERNEL_BATCH, 10, warmup)


ROOFLINE_TIMING = f"graph replay of {KERNEL_BATCH} back-to-back calls over the rotated pools, divided by {KERNEL_BATCH}"


def graph_step_ms(capture_fns, steps, warmup):
    """Capture each step variant (one per pool copy) into a HIP graph via
    torch.cuda.graph and time `steps` replays, cycling the variants.  Returns
    the wall milliseconds per step."""
    graphs = []
    for fn in capture_fns:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            fn()
        graphs.append(g)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    settle(lambda i: graphs[i % len(graphs)].replay())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def cpu_baseline_decode(step, write, budget_s):
    """Time the oracle (as is) on the step's inputs: KV write + decode of
    all sequences, repeated while the budget lasts (at least once)."""
    import oracle

    threads = torch.get_num_threads()
    t0 = time.perf_counter()
    passes = 0
    while True:
        kc, vc = step.k_cache, step.v_cache
        if write:
            kc, vc = oracle.kv_cache_write(step.new_k, step.new_v, step.slot_mapping, kc, vc)
        oracle.decode(step.decode_q, kc, vc, step.decode_block_tables, step.decode_context_lens, step.scale)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (passes + 1) / passes > 3 * budget_s:
            break
    per_pass = el / passes
    nbytes = W.decode_bytes(step) + (W.kv_write_bytes(step) if write else 0)
    # The same oracle on one thread, on the first sequences for about a tenth
    # of the budget, scaled by bytes.
    torch.set_num_threads(1)
    try:
        n1 = 0
        t1 = time.perf_counter()
        while n1 < step.num_decode and time.perf_counter() - t1 < budget_s / 10:
            n0, n1 = n1, min(step.num_decode, n1 + 8)
            oracle.decode(step.decode_q, step.k_cache, step.v_cache, step.decode_block_tables,
                          step.decode_context_lens, step.scale, seqs=list(range(n0, n1)))
        el1 = time.perf_counter() - t1
    finally:
        torch.set_num_threads(threads)
    one = W.decode_bytes(step, seqs=list(range(n1))) / el1 / 1e9
    return {
        "value": round(nbytes / per_pass / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 torch-CPU oracle: {'KV write + ' if write else ''}decode of all {step.num_decode} "
                  f"sequences, {passes} pass(es) in {el:.1f} s ({per_pass * 1e3:.0f} ms/pass), "
                  f"{os.cpu_count()} host CPUs visible ({cpu_model()})",
        "ms_per_step": round(per_pass * 1e3, 2),
        "single_thread_value": round(one, 4),
        "single_thread_sample": f"decode of the first {n1} sequences on 1 thread in {el1:.1f} s",
    }


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "cpu model unknown"


def bench_decode_step(args, pka):
    step = W.config_3(seed=args.seed)
    log(f"config3: {step.num_decode} seqs, {int(step.context_lens.sum())} context tokens, pool {step.num_blocks} blocks")
    P = Pools(step, args.rotate)
    S, Hq, D = step.decode_q.shape
    max_ctx = step.max_context_len
    variant = pka.decode_choose_variant(S, step.num_kv_heads, max_ctx)
    ws = pka.splitk_workspace(S, Hq, D, max_ctx, "cuda:0")

    # Comparison arm, timed first: the same step as two launches, the KV
    # write and then the dispatched decode reading the rows just written.
    separate = None
    if not args.no_arms:
        writes = [pka.kv_cache_write(P.new_k, P.new_v, P.slots, P.k[r], P.v[r], prepare=True) for r in range(P.R)]
        decs = [pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, max_ctx, out=P.out, workspace=ws,
                                      prepare=True) for r in range(P.R)]

        def launch2(i, ev):
            r = i % P.R
            if ev:
                ev[0].record()
            writes[r]()
            if ev:
                ev[1].record()
            decs[r]()
            if ev:
                ev[2].record()

        sep_wall, (write_ms, dec_ms) = timed_loop(launch2, 2, args.steps, args.warmup)
        separate = {"kv_write_us_per_call": round(write_ms * 1e3, 2), "decode_us_per_call": round(dec_ms * 1e3, 2),
                    "eager_ms_per_step": round(sep_wall, 4)}
        if not args.no_graph:
            def sep_fn(r):
                return lambda: (pka.kv_cache_write(P.new_k, P.new_v, P.slots, P.k[r], P.v[r]),
                                pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, max_ctx,
                                                      out=P.out, workspace=ws))
            separate["graph_ms_per_step"] = round(graph_step_ms([sep_fn(r) for r in range(P.R)], args.steps,
                                                                args.warmup), 4)

    # The step: one launch that writes each sequence's new K/V row at its
    # last position and decodes over the context including it.
    fused = [pka.paged_attn_decode_append(P.q, P.new_k, P.new_v, P.k[r], P.v[r], P.bt, P.cl, step.scale, max_ctx,
                                          out=P.out, workspace=ws, prepare=True) for r in range(P.R)]

    def launch(i, ev):
        r = i % P.R
        if ev:
            ev[0].record()
        fused[r]()
        if ev:
            ev[1].record()

    st = {}
    wall_ms, (fused_ms,) = timed_loop(launch, 1, args.steps, args.warmup, stats=st)
    eager_ms = wall_ms
    graph_ms = None
    if not args.no_graph:
        # The same step launched as a captured HIP graph (how a serving loop
        # replays its decode step); the captured calls read torch's capture stream.
        def step_fn(r):
            return lambda: pka.paged_attn_decode_append(P.q, P.new_k, P.new_v, P.k[r], P.v[r], P.bt, P.cl,
                                                        step.scale, max_ctx, out=P.out, workspace=ws)
        graph_ms = graph_step_ms([step_fn(r) for r in range(P.R)], args.steps, args.warmup)
        wall_ms = graph_ms
    dbytes = W.decode_bytes(step)
    wbytes = W.kv_write_bytes(step)
    value = (dbytes + wbytes) / (wall_ms * 1e-3) / 1e9
    kern_us = None
    if not args.no_graph:
        kern_us = back_to_back_us(lambda r: pka.paged_attn_decode_append(P.q, P.new_k, P.new_v, P.k[r], P.v[r], P.bt,
                                                                         P.cl, step.scale, max_ctx, out=P.out,
                                                                         workspace=ws), P.R, args.warmup)
    kern_ms = kern_us[1] * 1e-3 if kern_us else fused_ms
    achieved = (dbytes + wbytes) / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "paged decode µs/call + achieved HBM GB/s (% of 8 TB/s peak), 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(wall_ms, 4),
        "step_launch": "hip-graph replay" if graph_ms is not None else "eager",
        "eager_ms_per_step": round(eager_ms, 4),
        "decode_us_per_call": round(fused_ms * 1e3, 2),
        "decode_us_p10_p50_p90": [round(x * 1e3, 2) for x in st["pct"][0]],
        "kernel_us_back_to_back_p10_p50_p90": None if kern_us is None else [round(x, 2) for x in kern_us],
        "kv_write": "folded into the decode launch (pka_paged_attn_decode_append)",
        "separate_write_then_decode": separate,
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "dtype": "bf16",
        "config": {
            "workload": "batched GQA paged decode step (KV write of 256 rows + decode), bf16, 256 seqs, "
                        "16q/8kv heads, head_dim 128, block 16, ctx U[100,2048]",
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": step.num_kv_heads, "head_dim": D,
            "block_size": step.block_size, "context_tokens": int(step.context_lens.sum()),
            "max_context_len": max_ctx, "pool_blocks": step.num_blocks, "pool_copies_rotated": P.R,
            "decode_variant": "single-pass" if variant == 1 else "split-K (one launch)", "seed": args.seed,
            "algorithmic_bytes": {"decode": dbytes, "kv_write": wbytes},
        },
        "roofline": {
            "kernel": ("paged_decode_kernel (single pass, KV write folded in)" if variant == 1
                       else "split-K decode + reduce (KV write folded in)"),
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "timing": ROOFLINE_TIMING if kern_us else "HIP events around each call",
            "us_per_launch": round(kern_ms * 1e3, 2),
        },
    }
    return res, step, True


def bench_splitk(args, pka):
    step = W.config_4(seed=args.seed)
    P = Pools(step, args.rotate)
    S, Hq, D = step.decode_q.shape
    max_ctx = step.max_context_len
    assert pka.decode_choose_variant(S, step.num_kv_heads, max_ctx) == 2
    dbytes = W.decode_bytes(step)

    # Comparison arm, timed first: the same decode as two launches (the
    # partition pass, then the separate reduce kernel).
    two_launch = None
    if not args.no_arms:
        bufs = pka.splitk_buffers(S, Hq, D, max_ctx, "cuda:0")
        parts = [pka.paged_attn_decode_splitk(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, *bufs, prepare=True)
                 for r in range(P.R)]
        reduce = pka.paged_attn_splitk_reduce(*bufs, P.cl, P.out, prepare=True)

        def launch2(i, ev):
            r = i % P.R
            if ev:
                ev[0].record()
            parts[r]()
            if ev:
                ev[1].record()
            reduce()
            if ev:
                ev[2].record()

        wall2, (part_ms, red_ms) = timed_loop(launch2, 2, args.steps, args.warmup)
        two_launch = {"partition_us_per_call": round(part_ms * 1e3, 2), "reduce_us_per_call": round(red_ms * 1e3, 2),
                      "eager_ms_per_step": round(wall2, 4),
                      "partition_pass_gbs": round(dbytes / (part_ms * 1e-3) / 1e9, 1)}

    # The step: the dispatched decode - one launch whose last partition of
    # each (sequence, KV head) merges the partitions into the output.
    ws = pka.splitk_workspace(S, Hq, D, max_ctx, "cuda:0")
    decs = [pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, max_ctx, out=P.out, workspace=ws,
                                  prepare=True) for r in range(P.R)]

    def launch(i, ev):
        r = i % P.R
        if ev:
            ev[0].record()
        decs[r]()
        if ev:
            ev[1].record()

    st = {}
    wall_ms, (dec_ms,) = timed_loop(launch, 1, args.steps, args.warmup, stats=st)
    eager_ms = wall_ms
    graph_ms = None
    if not args.no_graph:
        def step_fn(r):
            return lambda: pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, max_ctx, out=P.out,
                                                 workspace=ws)
        graph_ms = graph_step_ms([step_fn(r) for r in range(P.R)], args.steps, args.warmup)
        wall_ms = graph_ms
    value = dbytes / (wall_ms * 1e-3) / 1e9
    kern_us = None
    if not args.no_graph:
        kern_us = back_to_back_us(lambda r: pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, max_ctx,
                                                                   out=P.out, workspace=ws), P.R, args.warmup)
    kern_ms = kern_us[1] * 1e-3 if kern_us else dec_ms
    achieved = dbytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "paged decode µs/call + achieved HBM GB/s (% of 8 TB/s peak), 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(wall_ms, 4),
        "step_launch": "hip-graph replay" if graph_ms is not None else "eager",
        "eager_ms_per_step": round(eager_ms, 4),
        "decode_us_per_call": round(dec_ms * 1e3, 2),
        "decode_us_p10_p50_p90": [round(x * 1e3, 2) for x in st["pct"][0]],
        "kernel_us_back_to_back_p10_p50_p90": None if kern_us is None else [round(x, 2) for x in kern_us],
        "two_launch_partition_then_reduce": two_launch,
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "dtype": "bf16",
        "config": {
            "workload": "split-K paged decode, bf16, 4 seqs x 16384 ctx, 16q/8kv, head_dim 128, 256-token partitions",
            "num_seqs": S, "num_q_heads": Hq, "num_kv_heads": step.num_kv_heads, "head_dim": D,
            "context_tokens": int(step.context_lens.sum()), "pool_copies_rotated": P.R, "seed": args.seed,
            "decode_variant": "split-K, one launch (last partition merges)",
            "algorithmic_bytes": {"decode": dbytes},
        },
        "roofline": {
            "kernel": "paged_decode_kernel (split-K partitions + in-kernel merge, one launch)", "bound": "hbm",
            "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
            "timing": ROOFLINE_TIMING if kern_us else "HIP events around each call",
            "us_per_launch": round(kern_ms * 1e3, 2),
        },
    }
    return res, step, False


def bench_mixed(args, pka):
    step = W.config_5(seed=args.seed)
    P = Pools(step, args.rotate)
    nd = step.num_decode
    S, Hq, D = step.decode_q.shape
    max_dec = int(step.decode_context_lens.max())
    ws = pka.splitk_workspace(S, Hq, D, max_dec, "cuda:0")
    qd, qp = P.q[:nd], P.q[nd:]
    od, op = P.out[:nd], P.out[nd:]
    btd, btp = P.bt[:nd], P.bt[nd:]
    cld, clp = P.cl[:nd], P.cl[nd:]
    mql = step.max_query_len
    mcl = int(step.prefill_context_lens.max())
    pws = pka.prefill_workspace(step.num_prefill, step.num_prefill_rows, Hq, step.num_kv_heads, D, mcl, "cuda:0")

    writes = [pka.kv_cache_write(P.new_k, P.new_v, P.slots, P.k[r], P.v[r], prepare=True) for r in range(P.R)]
    decs = [pka.paged_attn_decode(qd, P.k[r], P.v[r], btd, cld, step.scale, max_dec, out=od, workspace=ws,
                                  prepare=True) for r in range(P.R)]
    pres = [pka.paged_attn_prefill(qp, P.k[r], P.v[r], btp, clp, P.qsl, step.scale, mql, mcl, out=op, workspace=pws,
                                   prepare=True) for r in range(P.R)]
    # "Unified" comparison arm (mini_engine, "Custom CUDA kernels"): every row,
    # decodes included as one-row chunks, through the prefill kernel.  Timed
    # beside the step, not part of it.
    qsl_all = torch.cat([torch.arange(nd, dtype=torch.int32), nd + step.query_start_loc]).to(P.q.device)
    mcl_all = int(step.context_lens.max())
    uws = pka.prefill_workspace(S + step.num_prefill, P.q.shape[0], Hq, step.num_kv_heads, D, mcl_all, "cuda:0")
    uout = torch.empty_like(P.q)
    unis = [pka.paged_attn_prefill(P.q, P.k[r], P.v[r], P.bt, P.cl, qsl_all, step.scale, mql, mcl_all, out=uout,
                                   workspace=uws, prepare=True) for r in range(P.R)]

    def launch(i, ev):
        r = i % P.R
        if ev:
            ev[0].record()
        writes[r]()
        if ev:
            ev[1].record()
        decs[r]()
        if ev:
            ev[2].record()
        pres[r]()
        if ev:
            ev[3].record()
            if not args.no_arms:
                unis[r]()
            ev[4].record()

    # The wall clock covers the step only on warm-up passes (ev is None); the
    # timed passes also run the unified arm, so the step time is the event sum.
    _, (write_ms, dec_ms, pre_ms, uni_ms) = timed_loop(launch, 4, args.steps, args.warmup)
    eager_ms = write_ms + dec_ms + pre_ms
    wall_ms = eager_ms
    graph_ms = graph2_ms = None
    if not args.no_graph:
        # The step as a captured HIP graph (write, decode, prefill + merge),
        # one per pool copy, replayed in turn.
        def step_fn(r):
            return lambda: (pka.kv_cache_write(P.new_k, P.new_v, P.slots, P.k[r], P.v[r]),
                            pka.paged_attn_decode(qd, P.k[r], P.v[r], btd, cld, step.scale, max_dec, out=od,
                                                  workspace=ws),
                            pka.paged_attn_prefill(qp, P.k[r], P.v[r], btp, clp, P.qsl, step.scale, mql, mcl, out=op,
                                                   workspace=pws))
        graph_ms = graph_step_ms([step_fn(r) for r in range(P.R)], args.steps, args.warmup)
        wall_ms = graph_ms

        # Comparison arm: the same step with the HBM-bound decode forked onto a
        # second stream beside the MFMA-bound prefill (they write disjoint rows
        # of `out`), joined before the step ends, captured into one graph.
        side_g = torch.cuda.Stream(device=P.q.device)  # default priority

        def step_fn2(r):
            def fn():
                pka.kv_cache_write(P.new_k, P.new_v, P.slots, P.k[r], P.v[r])
                side_g.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(side_g):
                    pka.paged_attn_decode(qd, P.k[r], P.v[r], btd, cld, step.scale, max_dec, out=od, workspace=ws)
                pka.paged_attn_prefill(qp, P.k[r], P.v[r], btp, clp, P.qsl, step.scale, mql, mcl, out=op,
                                       workspace=pws)
                torch.cuda.current_stream().wait_stream(side_g)
            return fn
        # Comparison arm only: measured slower as a graph than the one-stream step.
        if not args.no_arms:
            graph2_ms = graph_step_ms([step_fn2(r) for r in range(P.R)], args.steps, args.warmup)
    dbytes = W.decode_bytes(step)
    wbytes = W.kv_write_bytes(step)
    pbytes = W.prefill_bytes(step)
    flops = W.prefill_flops(step)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    value = (dbytes + wbytes + pbytes) / (wall_ms * 1e-3) / 1e9
    ceiling = None if args.no_arms else gemm_ceiling_tflops()
    # The roofline's time: the prefill call (attention + split merge) back to back.
    kern_us = None
    if not args.no_graph:
        kern_us = back_to_back_us(lambda r: pka.paged_attn_prefill(qp, P.k[r], P.v[r], btp, clp, P.qsl, step.scale, mql,
                                                                   mcl, out=op, workspace=pws), P.R, args.warmup)
    kern_ms = kern_us[1] * 1e-3 if kern_us else pre_ms
    kern_tflops = flops / (kern_ms * 1e-3) / 1e12

    # Two-stream schedule of the same step (comparison arm): after the KV
    # write, the HBM-bound decode runs on a second stream beside the
    # MFMA-bound prefill (they write disjoint rows of `out`).
    two_ms = None
    if not args.no_arms:
        main = torch.cuda.current_stream()
        side = torch.cuda.Stream(device=P.q.device)
        with torch.cuda.stream(side):
            decs2 = [pka.paged_attn_decode(qd, P.k[r], P.v[r], btd, cld, step.scale, max_dec, out=od, workspace=ws,
                                           prepare=True) for r in range(P.R)]
        written = torch.cuda.Event()
        decoded = torch.cuda.Event()

        def launch2(i, ev):
            r = i % P.R
            if ev:
                ev[0].record(main)
            writes[r]()
            written.record(main)
            side.wait_event(written)
            decs2[r]()
            pres[r]()
            decoded.record(side)
            main.wait_event(decoded)
            if ev:
                ev[1].record(main)

        _, (two_ms,) = timed_loop(launch2, 1, args.steps, args.warmup)
    res = {
        "metric": "paged decode µs/call + achieved HBM GB/s (% of 8 TB/s peak), 1 MI355X",
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(wall_ms, 4),
        "step_launch": "hip-graph replay" if graph_ms is not None else "eager (event sum)",
        "graph_ms_per_step_one_stream": None if graph_ms is None else round(graph_ms, 4),
        "graph_ms_per_step_two_streams": None if graph2_ms is None else round(graph2_ms, 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "kv_write_us_per_call": round(write_ms * 1e3, 2),
        "decode_us_per_call": round(dec_ms * 1e3, 2),
        "decode_GBps": round(dbytes / (dec_ms * 1e-3) / 1e9, 1),
        "prefill_us_per_call": round(pre_ms * 1e3, 2),
        "prefill_TFLOPs": round(tflops, 1),
        "prefill_us_back_to_back_p10_p50_p90": None if kern_us is None else [round(x, 2) for x in kern_us],
        "unified_arm_us_per_call": None if args.no_arms else round(uni_ms * 1e3, 2),
        "unified_vs_split_attention": None if args.no_arms else round(uni_ms / (dec_ms + pre_ms), 2),
        "two_stream_ms_per_step": None if two_ms is None else round(two_ms, 4),
        "two_stream_GBps": None if two_ms is None else round((dbytes + wbytes + pbytes) / (two_ms * 1e-3) / 1e9, 2),
        "dtype": "bf16",
        "config": {
            "workload": "mixed paged step: KV write of 2048 rows, 64 decodes (ctx U[128,2048]) and ragged causal "
                        "prefill chunks (<=512 rows) into one output, bf16, 16q/8kv, head_dim 128, budget 2048",
            "decode_seqs": nd, "prefill_chunks": step.num_prefill, "prefill_rows": step.num_prefill_rows,
            "chunk_q_lens": step.meta["prefill_qlen"], "chunk_cached": step.meta["prefill_cached"],
            "pool_copies_rotated": P.R, "seed": args.seed,
            "algorithmic": {"decode_bytes": dbytes, "kv_write_bytes": wbytes, "prefill_bytes": pbytes,
                            "prefill_flops": flops},
        },
        "roofline": {
            "kernel": "paged_prefill_kernel + paged_prefill_merge_kernel (one prefill call)", "bound": "mfma",
            "achieved": round(kern_tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(kern_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
            "timing": ROOFLINE_TIMING if kern_us else "HIP events around each call",
            "us_per_launch": round(kern_ms * 1e3, 2),
            # What a plain library GEMM reaches on this GPU, beside the spec peak.
            "measured_ceiling": ceiling,
            "frac_of_measured_ceiling": None if ceiling is None else round(kern_tflops / ceiling["TFLOPs"], 4),
        },
    }
    return res, step, True


def gemm_ceiling_tflops(n=8192, reps=10):
    """bf16 dense GEMM rate of the vendor library (torch.matmul -> hipBLASLt),
    n x n x n, median of `reps` event-timed calls after warm-up."""
    a = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda:0").to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda:0", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        torch.matmul(a, b, out=c)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))[reps // 2]
    del a, b, c
    return {"TFLOPs": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1), "gemm": f"bf16 {n}x{n}x{n} torch.matmul"}


def bench_prefill_long(args, pka):
    """Prefill alone on long chunks: 4 sequences x 2,048 new rows after 6,144
    cached tokens (bf16, 16q/8kv, head_dim 128), one launch (attention + split
    merge).  MFMA-bound; the size where load balance no longer matters."""
    ql, cached = [2048] * 4, [6144] * 4
    step = W.make_prefill_step(query_lens=ql, cached_lens=cached, dtype=torch.bfloat16, num_q_heads=16,
                               num_kv_heads=8, head_dim=128, seed=args.seed, poison=False, write_new=False)
    dev = torch.device("cuda:0")
    k, v, q = step.k_cache.to(dev), step.v_cache.to(dev), step.q.to(dev)
    bt, cl, qsl = step.block_tables.to(dev), step.context_lens.to(dev), step.query_start_loc.to(dev)
    out = torch.empty_like(q)
    Hq, D, Hkv = q.shape[1], q.shape[2], step.num_kv_heads
    mcl = int(step.context_lens.max())
    ws = pka.prefill_workspace(step.num_prefill, step.num_prefill_rows, Hq, Hkv, D, mcl, dev)
    run = pka.paged_attn_prefill(q, k, v, bt, cl, qsl, step.scale, step.max_query_len, mcl, out=out, workspace=ws,
                                 prepare=True)

    def launch(i, ev):
        if ev:
            ev[0].record()
        run()
        if ev:
            ev[1].record()

    wall_ms, (pre_ms,) = timed_loop(launch, 1, args.steps, args.warmup)
    flops = W.prefill_flops(step)
    tflops = flops / (pre_ms * 1e-3) / 1e12
    ceiling = None if args.no_arms else gemm_ceiling_tflops()
    res = {
        "metric": "paged prefill TFLOP/s (bf16 MFMA, algorithmic FLOPs), 1 MI355X",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "ms_per_step": round(wall_ms, 4),
        "prefill_us_per_call": round(pre_ms * 1e3, 2),
        "dtype": "bf16",
        "config": {"workload": "paged prefill: 4 chunks of 2,048 rows after 6,144 cached tokens each, bf16, "
                               "16q/8kv, head_dim 128, block 16",
                   "query_lens": ql, "cached_lens": cached, "seed": args.seed,
                   "algorithmic": {"prefill_flops": flops, "prefill_bytes": W.prefill_bytes(step)}},
        "roofline": {
            "kernel": "paged_prefill_kernel", "bound": "mfma", "achieved": round(tflops, 1),
            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": None, "timing": "HIP events around each call (one launch: no split to merge)",
            "us_per_launch": round(pre_ms * 1e3, 2), "measured_ceiling": ceiling,
            "frac_of_measured_ceiling": None if ceiling is None else round(tflops / ceiling["TFLOPs"], 4),
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(step, args.cpu_seconds)
    return res, None, False


# (label, dtype, Hq, Hkv, head_dim, block) of the prefill shape rows: the
# long prefill's chunks (4 x 2,048 rows after 6,144 cached) at other head,
# group and block shapes.
PREFILL_SHAPES = [
    ("G2 d128 b16 (16q/8kv)", torch.bfloat16, 16, 8, 128, 16),
    ("G8 d128 b16 (32q/4kv)", torch.bfloat16, 32, 4, 128, 16),
    ("G4 d128 b32 (32q/8kv)", torch.bfloat16, 32, 8, 128, 32),
    ("G1 d128 b16 (16q/16kv, fp16)", torch.float16, 16, 16, 128, 16),
    ("G2 d64 b16 (32q/16kv)", torch.bfloat16, 32, 16, 64, 16),
    ("G2 d256 b8 (8q/4kv)", torch.bfloat16, 8, 4, 256, 8),
]


def bench_prefill_shapes(args, pka):
    """The prefill on the long prefill's chunks at each of PREFILL_SHAPES:
    us per call (events around each call) and algorithmic TFLOP/s."""
    ql, cached = [2048] * 4, [6144] * 4
    dev = torch.device("cuda:0")
    rows = {}
    first = None
    for label, dtype, hq, hkv, d, bs in PREFILL_SHAPES:
        step = W.make_prefill_step(query_lens=ql, cached_lens=cached, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                                   head_dim=d, block_size=bs, seed=args.seed, poison=False, write_new=False)
        k, v, q = step.k_cache.to(dev), step.v_cache.to(dev), step.q.to(dev)
        bt, cl, qsl = step.block_tables.to(dev), step.context_lens.to(dev), step.query_start_loc.to(dev)
        out = torch.empty_like(q)
        mcl = int(step.context_lens.max())
        ws = pka.prefill_workspace(step.num_prefill, step.num_prefill_rows, hq, hkv, d, mcl, dev)
        run = pka.paged_attn_prefill(q, k, v, bt, cl, qsl, step.scale, step.max_query_len, mcl, out=out,
                                     workspace=ws, prepare=True)

        def launch(i, ev):
            if ev:
                ev[0].record()
            run()
            if ev:
                ev[1].record()

        st = {}
        _, (pre_ms,) = timed_loop(launch, 1, args.steps, args.warmup, stats=st)
        flops = W.prefill_flops(step)
        tflops = flops / (pre_ms * 1e-3) / 1e12
        rows[label] = {"us_per_call": round(pre_ms * 1e3, 2), "us_p10_p50_p90": [round(x * 1e3, 2) for x in st["pct"][0]],
                       "algorithmic_flops": flops, "TFLOPs": round(tflops, 1),
                       "pct_of_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 1)}
        log(f"{label}: {rows[label]['us_per_call']} us, {rows[label]['TFLOPs']} TFLOP/s")
        if first is None:
            first = (label, pre_ms, tflops)
        del k, v, q, out, ws, run
        torch.cuda.empty_cache()
    label, pre_ms, tflops = first
    return {
        "metric": "paged prefill TFLOP/s (bf16 MFMA, algorithmic FLOPs), 1 MI355X",
        "value": round(tflops, 1),
        "unit": "TFLOP/s",
        "ms_per_step": round(pre_ms, 4),
        "per_shape": rows,
        "dtype": "bf16",
        "config": {"workload": "paged prefill: 4 chunks of 2,048 rows after 6,144 cached tokens each, per "
                               "head/group/block shape; value: " + label, "seed": args.seed},
        "roofline": {"kernel": f"paged_prefill_kernel ({label})", "bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None},
        "cpu_baseline": None,
    }, None, False


def cpu_baseline_prefill(step, budget_s):
    """The oracle (as is) on a sample of the workload: rows of chunk 0 (each
    sees the 6,144 cached keys plus its causal prefix), as many as the budget
    allows, at least one; rate in algorithmic TFLOP/s."""
    import oracle

    threads = torch.get_num_threads()
    Hq, D = step.q.shape[1], step.q.shape[2]
    cached = int(step.context_lens[0]) - int(step.query_start_loc[1])
    t0 = time.perf_counter()
    rows = 0
    flops = 0
    while True:
        oracle.prefill(step.q, step.k_cache, step.v_cache, step.block_tables, step.context_lens,
                       step.query_start_loc, step.scale, seqs=[0], rows=[rows])
        flops += 4 * D * Hq * (cached + rows + 1)
        rows += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 torch-CPU oracle: the first {rows} rows of chunk 0 (6,144+ keys each) in {dt:.1f} s, "
                      f"{threads} host threads"}


def bench_sweep(args, pka, contexts=(128, 1024, 4096), name="sweep"):
    rows = {}
    last = None
    for ctx in contexts:
        step = W.config_1(seed=args.seed) if name == "single" else W.config_2(ctx, seed=args.seed)
        P = Pools(step, args.rotate or 2)
        S, Hq, D = step.decode_q.shape
        ws = pka.splitk_workspace(S, Hq, D, ctx, "cuda:0")

        decs = [pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, ctx, out=P.out, workspace=ws,
                                      prepare=True) for r in range(P.R)]

        def launch(i, ev):
            r = i % P.R
            if ev:
                ev[0].record()
            decs[r]()
            if ev:
                ev[1].record()

        st = {}
        wall_ms, (dec_ms,) = timed_loop(launch, 1, args.steps, args.warmup, stats=st)
        p10, p50, p90 = st["pct"][0]

        # Back-to-back: SWEEP_BATCH calls on one stream captured as one HIP
        # graph, each replay timed with events and divided by the batch, so
        # the figure is the device time per call (kernel plus the gap between
        # dependent launches), without host launch overhead.
        def batch():
            for i in range(SWEEP_BATCH):
                r = i % P.R
                pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, ctx, out=P.out, workspace=ws)

        batch_us = graph_batch_us(batch, SWEEP_BATCH, max(10, args.steps // 5), args.warmup)

        # Cold: a 512 MiB write between calls pushes the pool out of the L2s
        # and the Infinity Cache; the events bracket the decode alone.
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda:0")

        def cold(i, ev):
            flush.fill_(i & 0xFF)
            launch(i, ev)

        _, (cold_ms,) = timed_loop(cold, 1, args.steps, args.warmup)
        del flush

        # Materialise-then-attend arm: gather the request's pages into
        # contiguous K/V, then plain torch attention (the pages' comparison
        # path).  Every right-hand matmul operand is made contiguous first.
        nb = ctx // step.block_size
        tbl = P.bt[0, :nb].long()
        qh = P.q[0][:, None, :].contiguous()

        def mat(i, ev):
            r = i % P.R
            if ev:
                ev[0].record()
            kt = P.k[r].index_select(0, tbl).reshape(ctx, step.num_kv_heads, D).permute(1, 2, 0).contiguous()
            v = P.v[r].index_select(0, tbl).reshape(ctx, step.num_kv_heads, D).transpose(0, 1).contiguous()
            if ev:
                ev[1].record()
            p = torch.softmax(torch.matmul(qh, kt).float() * step.scale, dim=-1).to(v.dtype)
            torch.matmul(p, v)
            if ev:
                ev[2].record()

        mwall, (gather_ms, sdpa_ms) = timed_loop(mat, 2, args.steps, args.warmup)
        rows[str(ctx)] = {
            "decode_us_per_call": round(batch_us[1], 3),
            "decode_us_per_call_p10_p50_p90": [round(x, 3) for x in batch_us],
            "per_call_timing": f"graph replay of {SWEEP_BATCH} back-to-back calls, divided by {SWEEP_BATCH}",
            "single_call_event_us_p10_p50_p90": [round(x * 1e3, 2) for x in (p10, p50, p90)],
            "decode_cold_us_per_call": round(cold_ms * 1e3, 2),
            "decode_wall_us_per_call": round(wall_ms * 1e3, 2),
            "achieved_GBps": round(W.decode_bytes(step) / (batch_us[1] * 1e-6) / 1e9, 2),
            "materialise_then_attend_us": round(mwall * 1e3, 2),
            "materialise_gather_us": round(gather_ms * 1e3, 2),
            "variant": "single-pass" if pka.decode_choose_variant(S, step.num_kv_heads, ctx) == 1 else "split-K",
        }
        last = (step, batch_us[1] * 1e-3)
    step, call_ms = last
    value = W.decode_bytes(step) / (call_ms * 1e-3) / 1e9
    res = {
        "metric": "paged decode µs/call + achieved HBM GB/s (% of 8 TB/s peak), 1 MI355X",
        "value": round(value, 3),
        "unit": "GB/s",
        "ms_per_step": round(call_ms, 6),
        "per_context": rows,
        "dtype": "fp16",
        "config": {"workload": f"single-request fp16 paged decode, 2 heads, head_dim 64, block 16, ctx {list(contexts)}",
                   "seed": args.seed},
        "roofline": {
            "kernel": "paged decode (largest context)", "bound": "hbm",
            "achieved": round(W.decode_bytes(step) / (call_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(W.decode_bytes(step) / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 6),
            "traffic": None,
        },
    }
    return res, step, False


# Head and block shapes beyond the measured configs, each the decode step of
# config 3's batch (contexts uniform in [100, 2048]) with that shape:
# (label, dtype, q heads, KV heads, head size, block size).
DECODE_SHAPES = [
    ("G8 d128 b16 (64q/8kv)", torch.bfloat16, 64, 8, 128, 16),
    ("G4 d128 b16 (32q/8kv)", torch.bfloat16, 32, 8, 128, 16),
    ("G1 d128 b16 (32q/32kv, fp16)", torch.float16, 32, 32, 128, 16),
    ("G2 d128 b32 (16q/8kv)", torch.bfloat16, 16, 8, 128, 32),
    ("G2 d256 b32 (16q/8kv)", torch.bfloat16, 16, 8, 256, 32),
    ("G8 d256 b32 (32q/4kv)", torch.bfloat16, 32, 4, 256, 32),
    ("G8 d64 b16 (64q/8kv, fp16)", torch.float16, 64, 8, 64, 16),
]


def bench_shapes(args, pka):
    """The dispatched decode (single pass at this batch) on each of
    DECODE_SHAPES: us per call (events around each call, pools rotated) and
    achieved GB/s of the algorithmic bytes."""
    rows = {}
    first = None
    for label, dtype, hq, hkv, d, bs in DECODE_SHAPES:
        rng = np.random.default_rng(args.seed)
        n = 256 if hkv * d <= 1024 else 128
        ctx = [int(x) for x in rng.integers(100, 2049, size=n)]
        step = W.make_decode_step(context_lens=ctx, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                                  block_size=bs, seed=args.seed)
        P = Pools(step, args.rotate)
        S, Hq, D = step.decode_q.shape
        max_ctx = int(step.decode_context_lens.max())
        ws = pka.splitk_workspace(S, Hq, D, max_ctx, "cuda:0")
        decs = [pka.paged_attn_decode(P.q, P.k[r], P.v[r], P.bt, P.cl, step.scale, max_ctx, out=P.out, workspace=ws,
                                      prepare=True) for r in range(P.R)]

        def launch(i, ev):
            if ev:
                ev[0].record()
            decs[i % P.R]()
            if ev:
                ev[1].record()

        st = {}
        _, (dec_ms,) = timed_loop(launch, 1, args.steps, args.warmup, stats=st)
        gbs = W.decode_bytes(step) / (dec_ms * 1e-3) / 1e9
        rows[label] = {"num_seqs": n, "context_tokens": int(sum(ctx)), "us_per_call": round(dec_ms * 1e3, 2),
                       "us_p10_p50_p90": [round(x * 1e3, 2) for x in st["pct"][0]],
                       "algorithmic_bytes": W.decode_bytes(step), "achieved_GBps": round(gbs, 1),
                       "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                       "variant": "single-pass" if pka.decode_choose_variant(S, hkv, max_ctx) == 1 else "split-K"}
        log(f"{label}: {rows[label]['us_per_call']} us, {rows[label]['achieved_GBps']} GB/s")
        if first is None:
            first = (label, dec_ms, gbs)
        del P, decs, ws
        torch.cuda.empty_cache()
    label, dec_ms, gbs = first
    res = {
        "metric": "paged decode µs/call + achieved HBM GB/s (% of 8 TB/s peak), 1 MI355X",
        "value": round(gbs, 3),
        "unit": "GB/s",
        "ms_per_step": round(dec_ms, 5),
        "per_shape": rows,
        "dtype": "bf16",
        "config": {"workload": "decode of 256 (128 for the largest rows) sequences with contexts uniform in "
                               "[100, 2048], per head/block shape; value: " + label, "seed": args.seed},
        "roofline": {"kernel": f"paged_decode_kernel ({label})", "bound": "hbm", "achieved": round(gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None},
        "cpu_baseline": None,
    }
    return res, None, False


def cpu_baseline_rope(step, budget_s, rows=256):
    """Time the oracle (as is) on the first `rows` new rows of the step."""
    import oracle

    qkv = W.fused_qkv(step)[:rows]
    pos, slots = step.positions[:rows], step.slot_mapping[:rows]
    threads = torch.get_num_threads()
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.fused_rope_kv_write(qkv, pos, slots, step.k_cache, step.v_cache, step.num_q_heads, step.num_kv_heads,
                                   ROPE_THETA)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (passes + 1) / passes > 3 * budget_s:
            break
    per_pass = el / passes
    e = step.q.element_size()
    D, Hq, Hkv = step.head_dim, step.num_q_heads, step.num_kv_heads
    nbytes = rows * ((Hq + 2 * Hkv) * D * e + 16 + D * 4 + Hq * D * e + 2 * Hkv * D * e)
    return {
        "value": round(nbytes / per_pass / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"fp64 torch-CPU oracle: fused rotary + KV write of the first {rows} of {step.q.shape[0]} rows "
                  f"(the pool is cloned once per call), {passes} pass(es) in {el:.1f} s",
        "ms_per_step": round(per_pass * 1e3, 2),
    }


def bench_rope(args, pka):
    """Fused rotary + KV write of the mixed step's 2,048 new rows, next to the
    eager arm it replaces (torch rotation of q and k, then the KV write)."""
    step = W.config_5(seed=args.seed)
    dev = torch.device("cuda:0")
    T, Hq, D = step.q.shape
    Hkv = step.num_kv_heads
    max_pos = 8192
    assert int(step.positions.max()) < max_pos
    qkv = W.fused_qkv(step).to(dev)
    pos = step.positions.to(dev)
    slots = step.slot_mapping.to(dev)
    kc, vc = step.k_cache.to(dev), step.v_cache.to(dev)
    table = pka.rope_table(max_pos, D, ROPE_THETA, dev)
    q_out = torch.empty((T, Hq, D), dtype=step.dtype, device=dev)
    fused = pka.fused_rope_kv_write(qkv, pos, slots, table, Hq, kc, vc, q_out=q_out, prepare=True)

    rows = qkv.view(T, Hq + 2 * Hkv, D)
    cs = table[pos]  # [T, D/2, 2]
    cos, sin = cs[..., 0].unsqueeze(1), cs[..., 1].unsqueeze(1)

    def eager():
        x = rows[:, :Hq + Hkv].float()
        lo, hi = x[..., :D // 2], x[..., D // 2:]
        rot = torch.cat([lo * cos - hi * sin, hi * cos + lo * sin], dim=-1).to(step.dtype)
        q_out.copy_(rot[:, :Hq])
        pka.kv_cache_write(rot[:, Hq:].contiguous(), rows[:, Hq + Hkv:].contiguous(), slots, kc, vc)

    def launch(i, ev):
        if ev:
            ev[0].record()
        fused()
        if ev:
            ev[1].record()
        if not args.no_arms:
            eager()
        if ev:
            ev[2].record()

    wall_ms, (fused_ms, eager_ms) = timed_loop(launch, 2, args.steps, args.warmup)
    nbytes = W.rope_kv_write_bytes(step)
    gbps = nbytes / (fused_ms * 1e-3) / 1e9
    res = {
        "metric": "fused rotary + KV-cache write GB/s (% of 8 TB/s peak), 1 MI355X",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "ms_per_step": round(fused_ms, 4),
        "fused_us_per_call": round(fused_ms * 1e3, 2),
        "eager_arm_us_per_call": None if args.no_arms else round(eager_ms * 1e3, 2),
        "dtype": "bf16",
        "config": {
            "workload": "fused rotary embedding + KV-cache write of the mixed step's 2048 new rows, bf16, 16q/8kv, "
                        "head_dim 128, rotate-half RoPE, theta 1e6",
            "rows": T, "max_position": max_pos, "seed": args.seed, "algorithmic_bytes": nbytes,
            "eager_arm": "torch fp32 rotation of q and k + separate KV write (the pass the fusion removes)",
        },
        "roofline": {"kernel": "rope_kv_write_kernel", "bound": "hbm", "achieved": round(gbps, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline_rope(step, args.cpu_seconds)
    return res, None, False


def block_manager_trace(seed, steps, budget=2048, num_blocks=20000, block_size=16):
    """A chunked-prefill serving trace as host operations: each step
    schedules the running decodes, then continues or admits prompts in chunks
    until the token budget is used (prompts 90% U[128,512] / 10% U[4096,7680],
    30% sharing one 256-token prefix, outputs U[16,256] tokens)."""
    rng = np.random.default_rng(seed)
    prefix = rng.integers(0, 150000, size=256).tolist()
    ops, rid = [], 0
    live = {}  # rid -> [prompt_len, computed, to_generate]
    waiting = []
    for _ in range(steps):
        left = budget
        step = []
        for r in list(live):
            plen, comp, gen = live[r]
            if comp >= plen and left > 0:  # decode
                step.append(("decode", r))
                left -= 1
                live[r][2] -= 1
                if live[r][2] <= 0:
                    step.append(("finish", r))
                    del live[r]
        while left > 0:
            if not waiting:
                rid += 1
                P = int(rng.integers(4096, 7681)) if rng.random() < 0.1 else int(rng.integers(128, 513))
                toks = (prefix if rng.random() < 0.3 and P > 256 else []) + rng.integers(0, 150000, size=P).tolist()
                waiting.append((rid, toks, int(rng.integers(16, 257))))
            r, toks, gen = waiting.pop(0)
            n = min(len(toks), left, 512)
            step.append(("admit", r, toks, n))
            left -= n
            if n < len(toks):
                step.append(("chunks", r, len(toks) - n))
            live[r] = [len(toks), len(toks), gen]
        ops.append(step)
    return ops, num_blocks, block_size


def run_block_manager_trace(mgr, ops, rng_seed=0):
    """Replay a trace through a manager (library or reference); returns the
    number of tokens scheduled.  A step's decodes go through one batched call
    when the manager has it."""
    rng = np.random.default_rng(rng_seed)
    tokens = 0
    alive = set()  # admitted requests (the trace was drawn without knowing which fit)
    batched = hasattr(mgr, "decode_step")
    for step in ops:
        dec = [op[1] for op in step if op[0] == "decode" and op[1] in alive]
        toks = rng.integers(0, 150000, size=len(dec)).tolist()
        if batched and dec:
            _, ok = mgr.decode_step(dec, toks)
            tokens += int(ok.sum())
        else:
            for r, t in zip(dec, toks):
                mgr.append_token(r, t)
                if mgr.allocate(r, 1):
                    mgr.commit(r, 1)
                    tokens += 1
        for op in step:
            kind, r = op[0], op[1]
            if kind == "finish" and r in alive:
                mgr.free_request(r)
                alive.discard(r)
            elif kind == "admit":
                toks, n = op[2], op[3]
                mgr.add_request(r, toks)
                cached = mgr.admit(r, n)
                if cached is None:
                    mgr.free_request(r)
                    continue
                alive.add(r)
                step_n = min(n, len(toks) - cached)
                mgr.commit(r, step_n)
                tokens += step_n
                rest = len(toks) - cached - step_n
                while rest > 0:  # later chunks of the same prompt
                    c = min(rest, 512)
                    if not mgr.allocate(r, c):
                        break
                    mgr.commit(r, c)
                    tokens += c
                    rest -= c
    return tokens


def bench_block_manager(args, pka):
    """Host workload on the same data structure the kernels read: the
    library's C++ block manager replaying a chunked-prefill serving trace."""
    ops, N, B = block_manager_trace(args.seed, max(args.steps, 1) * 20)
    warm = pka.BlockManager(N, B)
    run_block_manager_trace(warm, ops[: max(1, len(ops) // 10)])
    mgr = pka.BlockManager(N, B)
    t0 = time.perf_counter()
    tokens = run_block_manager_trace(mgr, ops)
    el = time.perf_counter() - t0
    res = {
        "metric": "block-manager scheduled tokens/s (host, one core)",
        "value": round(tokens / el, 1),
        "unit": "tokens/s",
        "ms_per_step": round(el * 1e3 / len(ops), 4),
        "higher_is_better": True,
        "dtype": "int32",
        "config": {"workload": f"chunked-prefill serving trace through the C++ block manager: {len(ops)} steps of "
                               f"budget 2048, {N} pages of {B} tokens, prompts 90% U[128,512] / 10% U[4096,7680], "
                               "30% sharing a 256-token prefix", "tokens": tokens, "seed": args.seed},
        "roofline": None,
    }
    if not args.no_cpu_baseline:
        from oracle.block_manager import RefBlockManager

        sample = ops[: max(1, len(ops) // 4)]
        ref = RefBlockManager(N, B)
        t0 = time.perf_counter()
        rt = run_block_manager_trace(ref, sample)
        rel = time.perf_counter() - t0
        res["cpu_baseline"] = {"value": round(rt / rel, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"the Python reference manager on the first {len(sample)} steps "
                                         f"({rt} tokens in {rel:.2f} s)"}
    return res, None, False


def bench_copy(args):
    """Calibration: a plain device-to-device copy of 1 GiB (known read and
    write bytes), the reference against which the HBM traffic counters of the
    attention kernels are scaled."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)

    def launch(i, ev):
        if ev:
            ev[0].record()
        dst.copy_(src)
        if ev:
            ev[1].record()

    wall_ms, (copy_ms,) = timed_loop(launch, 1, args.steps, args.warmup)
    res = {
        "metric": "device-to-device copy GB/s (read + write), calibration",
        "value": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "ms_per_step": round(wall_ms, 4),
        "dtype": "u8",
        "config": {"workload": "copy of 1 GiB (1,048,576 KiB read + 1,048,576 KiB written per launch)"},
        "roofline": {"kernel": "torch copy", "bound": "hbm", "achieved": round(2 * n / (copy_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(2 * n / (copy_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4), "traffic": None},
    }
    return res, None, False


def main():
    global SETTLE_S
    args = parse_args()
    SETTLE_S = max(0.0, args.settle_ms / 1e3)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "this library has no multi-GPU path.", flush=True)
        sys.exit(2)
    host_only = args.workload == "block_manager"  # host data structure, no kernels
    if not host_only and not torch.cuda.is_available():
        print("bench.py needs a GPU", flush=True)
        sys.exit(1)
    import paged_kv_attention_21_amd as pka

    if torch.cuda.is_available():
        torch.cuda.set_device(0)
    if args.workload == "decode_step":
        res, step, write = bench_decode_step(args, pka)
    elif args.workload == "splitk":
        res, step, write = bench_splitk(args, pka)
    elif args.workload == "sweep":
        res, step, write = bench_sweep(args, pka)
    elif args.workload == "mixed":
        res, step, write = bench_mixed(args, pka)
    elif args.workload == "copy":
        res, step, write = bench_copy(args)
    elif args.workload == "single":
        res, step, write = bench_sweep(args, pka, contexts=(128,), name="single")
    elif args.workload == "rope_kv_write":
        res, step, write = bench_rope(args, pka)
    elif args.workload == "block_manager":
        res, step, write = bench_block_manager(args, pka)
    elif args.workload == "prefill_long":
        res, step, write = bench_prefill_long(args, pka)
    elif args.workload == "shapes":
        res, step, write = bench_shapes(args, pka)
    elif args.workload == "prefill_shapes":
        res, step, write = bench_prefill_shapes(args, pka)
    else:
        raise SystemExit(f"workload {args.workload} is not available yet")

    out = {
        "metric": res.pop("metric"),
        "value": res.pop("value"),
        "unit": res.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": res.pop("dtype"),
        "data": "synthetic (seeded N(0,1) q/K/V, seeded block tables and lengths)",
        "settle_s": SETTLE_S,
    }
    out.update(res)
    if isinstance(out.get("roofline"), dict):
        out["roofline"]["traffic"], out["roofline"]["traffic_source"] = recorded_traffic(args.workload)
    if "cpu_baseline" in out:
        pass  # the workload timed its own oracle sample
    elif not args.no_cpu_baseline and step is not None:
        log("timing the CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline_decode(step, write, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    out["gpu"] = fingerprint() if torch.cuda.is_available() else None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
