#!/usr/bin/env python3
"""Benchmark of the KDA training recurrence on one MI355X.

Workload: packed 8 x 1024 tokens, Hqk = Hv = 96, K = V = 128 (synthetic,
seeded; the FlashInfer page "flashinfer.kda_training" validates its kernels
on this exact shape).  A step is one pass of the hot path over that batch:
the training forward (o, final state and the FP32 state tape) followed by
the backward (all eight gradients) when --no-bwd is not given.

Printed: one JSON line with the forward throughput in token-heads/s (the
headline), the forward and backward times per step, the roofline of the
dominant kernel (the chunked forward) measured with HIP events on its own
stream, and the FP64 oracle timed on this host's cores as a CPU baseline.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "KDA fwd token-heads/sec (packed 8x1024, 96 heads, 1 GPU); % roofline; bwd time"
# HBM traffic of the chunked forward from rocprofv3 FETCH_SIZE / WRITE_SIZE
# passes, scaled by a copy kernel of known size; valid only for the kernel
# sources it was taken with (their SHA-256 is recorded beside the figures).
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_chunk_kernel_packed_8x1024_h96_traffic.txt")
FWD_SOURCES = ["gated_delta_rule_32_amd/csrc/kda_fwd_chunk.hip",
               "gated_delta_rule_32_amd/csrc/kda_chunk.hpp",
               "gated_delta_rule_32_amd/csrc/kda_common.hpp",
               "gated_delta_rule_32_amd/csrc/kda_kernels.h"]


ROUTE_NAMES = {1: "chunk", 2: "rowsplit", 3: "segments", 4: "chunk-split"}
ROUTE_KERNELS = {1: "fwd_chunk_kernel", 2: "fwd_rowsplit_kernel",
                 3: "fwd_chunk_kernel over all tape segments (P and Q, seg_combine_kernel, rerun): "
                    "the whole forward's time",
                 4: "fwd_chunk_kernel with the value columns split over two workgroups per task"}


def fwd_source_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in FWD_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic():
    """Measured HBM bytes per launch of the chunked forward, or None when no
    measurement exists for the current kernel sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for line in open(TRAFFIC_FILE):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256") != fwd_source_sha():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_fwd_bytes(problem) -> int:
    """Bytes the forward must move at least: q, k (shared by G heads), v, g,
    beta, o per token-head, plus the initial and final FP32 state per task."""
    toks = sum(problem.lengths)
    G = problem.Hv // problem.Hqk
    per_tok_head = 2 * 128 * 2 / G + 128 * 2 * 3 + 2
    return int(toks * problem.Hv * per_tok_head + problem.N * problem.Hv * 2 * 128 * 128 * 4)


def algorithmic_bwd_bytes(problem) -> int:
    """Bytes the backward must move at least: q, k (shared by G heads), v, g,
    beta, do read and dq, dk, dv, dg, dbeta written per token-head; the
    initial state and dfinal_state read and dinitial_state written per task."""
    toks = sum(problem.lengths)
    G = problem.Hv // problem.Hqk
    per_tok_head = 4 * 128 * 2 / G + 128 * 2 * 5 + 2 * 2
    return int(toks * problem.Hv * per_tok_head + problem.N * problem.Hv * 3 * 128 * 128 * 4)


def copy_calibration(nbytes: int = 1 << 30, reps: int = 5):
    """Plain device-to-device copies of a known size, to scale the HBM byte
    counters (run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE)."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_copy": nbytes, "copies": reps}), flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def copy_bandwidth(stream, nbytes: int = 1 << 30, reps: int = 10) -> float:
    """GB/s (bytes read plus bytes written) of a plain 1 GiB device copy,
    timed with HIP events on `stream`: the practical HBM ceiling of this GPU
    in this job, next to the nominal 8 TB/s."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").uniform_()
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(inp, max_seconds: float = 30.0):
    import numpy as np
    import oracle
    p = inp.problem
    workers = oracle.default_workers()
    # bounded sample: whole sequences x heads until ~max_seconds of estimated work
    est_per_tok_head = 60e-6
    budget = max_seconds * workers
    tasks = []
    work = 0.0
    for h in range(p.Hv):
        for n in range(p.N):
            if work >= budget:
                break
            tasks.append((n, h))
            work += p.lengths[n] * est_per_tok_head
    th = sum(p.lengths[n] for (n, h) in tasks)
    t = time.perf_counter()
    oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.A_log, inp.dt_bias,
                   inp.initial_state, p.lengths, p.packed, tasks=tasks, workers=workers)
    dt = time.perf_counter() - t
    return {"value": th / dt, "unit": "token-heads/s", "cores": workers, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"FP64 oracle forward of {len(tasks)} of {p.N * p.Hv} (sequence, head) "
                      f"tasks = {th} token-heads, {dt:.2f} s wall on {workers} processes"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="packed")
    ap.add_argument("--no-bwd", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--route", type=int, default=0)
    ap.add_argument("--ramp-ms", type=float, default=300.0,
                    help="untimed steps run first for this long, so the GPU reaches its "
                         "sustained clocks before the warm-up and timed steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain copies of 1 GiB (counter calibration)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="size of the buffer read before each launch of the secondary "
                         "cache-cold forward line (the main step needs none: each forward "
                         "follows the previous step's backward, which moves more than 2 GB "
                         "and so leaves nothing of the forward's inputs in L2 or the 256 MB "
                         "Infinity Cache)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the secondary lines (other workloads, tape-less forward, "
                         "cold plan, inference, records context)")
    ap.add_argument("--infer-only", action="store_true",
                    help="only time kda_infer (decode and prefill) on the packed workload's heads, "
                         "for per-kernel profiles of the inference routes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import workloads
    import gated_delta_rule_32_amd as kda

    inp_cpu = workloads.make_workload(args.workload, with_adjoints=True)
    p = inp_cpu.problem
    d = inp_cpu.to("cuda")
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    if args.infer_only:
        print(json.dumps({"inference": inference_steps(kda, p, d, inp_cpu, args, stream)}), flush=True)
        return
    prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp_cpu.cu_seqlens,
                            route=args.route)
    route, ntasks, _ = kda.kda_plan_query(prob)
    o = torch.empty_like(d.v)
    fs = torch.empty_like(d.initial_state)
    ctx = torch.empty(kda.kda_fwd_ctx_bytes(prob), dtype=torch.uint8, device=dev)
    do_bwd = not args.no_bwd
    if do_bwd:
        ws = torch.empty(kda.kda_bwd_workspace_bytes(prob), dtype=torch.uint8, device=dev)
        grads = (torch.empty_like(d.q), torch.empty_like(d.k), torch.empty_like(d.v),
                 torch.empty_like(d.g), torch.empty_like(d.beta), torch.empty_like(d.A_log),
                 torch.empty_like(d.dt_bias), torch.empty_like(d.initial_state))
    h = stream.cuda_stream

    def fwd():
        kda.kda_fwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                    o, fs, ctx, h)

    def bwd():
        kda.kda_bwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                    ctx, d.do, d.dfinal_state, *grads, ws, h)

    # clock ramp: the GPU raises its clocks only under sustained load (a few
    # warm-up steps leave the forward ~15% slower than in a training loop)
    ramp_steps = 0
    t_ramp = time.perf_counter()
    while (time.perf_counter() - t_ramp) * 1e3 < args.ramp_ms:
        for _ in range(4):
            fwd()
            if do_bwd:
                bwd()
        ramp_steps += 4
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        fwd()
        if do_bwd:
            bwd()
    torch.cuda.synchronize()

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        fwd()
        ev[i][1].record(stream)
        if do_bwd:
            bwd()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd_ms = sorted(a.elapsed_time(b) for a, b, _ in ev)
    bwd_ms = sorted(b.elapsed_time(c) for _, b, c in ev)
    fwd_med = fwd_ms[len(fwd_ms) // 2]
    fwd_mean = sum(fwd_ms) / len(fwd_ms)
    bwd_med = bwd_ms[len(bwd_ms) // 2]
    token_heads = p.token_heads
    value = token_heads / (fwd_mean * 1e-3)
    ms_per_step = wall * 1e3 / args.steps

    algo = algorithmic_fwd_bytes(p)
    achieved = algo / (fwd_mean * 1e-3) / 1e9
    traffic = recorded_traffic() if (route == 1 and p.name == "packed") else None
    copy_gbs = copy_bandwidth(stream)
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": ROUTE_KERNELS.get(route, "?"),
            "algorithmic_bytes_per_launch": algo, "avg_launch_ms": round(fwd_mean, 4),
            "copy_GBs_same_job": round(copy_gbs, 1),
            "frac_of_copy": round(achieved / copy_gbs, 4),
            "timed_after": "the previous step's backward (no explicit flush)"}
    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "token-heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp": {"ms": args.ramp_ms, "steps": ramp_steps},
        "ms_per_step": round(ms_per_step, 4),
        "fwd_ms_median": round(fwd_med, 4),
        "fwd_ms_p10": round(fwd_ms[len(fwd_ms) // 10], 4),
        "fwd_ms_p90": round(fwd_ms[(9 * len(fwd_ms)) // 10], 4),
        "bwd_ms_median": round(bwd_med, 4) if do_bwd else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{p.name}: {p.N} sequences x {p.lengths[0] if p.name != 'mixed' else 'mixed'}"
                               f" tokens, Hqk={p.Hqk}, Hv={p.Hv}, K=V=128",
                   "token_heads": token_heads, "route": ROUTE_NAMES.get(route, "?"),
                   "tape_interval": 256, "step": "fwd+bwd" if do_bwd else "fwd"},
        "roofline": roof,
    }
    if do_bwd:
        bwd_mean = sum(bwd_ms) / len(bwd_ms)
        ab = algorithmic_bwd_bytes(p)
        out["bwd"] = {"ms_mean": round(bwd_mean, 4),
                      "algorithmic_bytes": ab,
                      "achieved_GBs": round(ab / (bwd_mean * 1e-3) / 1e9, 1),
                      "frac_of_hbm_peak": round(ab / (bwd_mean * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                      "kernels": ["fwd_chunk_kernel<rebuild>", "bwd_chunk_kernel",
                                  "bwd_param_reduce_kernel", "bwd_dqk_reduce_kernel"]}
        if route == 1 and not args.no_extra:
            out["records_context"] = records_context_step(kda, p, d, inp_cpu, args, stream)
    if not args.no_extra:
        flush = torch.zeros(max(args.flush_mb, 0) << 18, dtype=torch.float32, device=dev)
        out["fwd_tapeless"] = tapeless_forward(kda, p, d, inp_cpu, args, stream, None)
        out["fwd_cache_cold"] = cache_cold_forward(kda, prob, p, d, args, stream, flush)
        del flush
        out["cold_plan"] = cold_plan_call(kda, p, d, inp_cpu, stream)
        if route in (0, 1):
            out["precision_cost"] = precision_cost(kda, p, d, inp_cpu, args, stream)
    if p.name == "packed" and not args.no_extra:
        out["inference"] = inference_steps(kda, p, d, inp_cpu, args, stream)
        out["other_workloads"] = other_workloads(kda, args, stream)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(inp_cpu)
    print(json.dumps(out), flush=True)


def _fwd_bwd_times(kda, prob, d, stream, steps, warmup, flush=None, bwd=True, ctx_none=False):
    """Mean forward and backward milliseconds by HIP events on `stream`."""
    import torch
    o = torch.empty_like(d.v)
    fs = torch.empty_like(d.initial_state)
    ctx = None if ctx_none else torch.empty(kda.kda_fwd_ctx_bytes(prob), dtype=torch.uint8,
                                            device="cuda")
    if bwd:
        ws = torch.empty(kda.kda_bwd_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
        grads = [torch.empty_like(t) for t in (d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias,
                                               d.initial_state)]
    h = stream.cuda_stream
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    flush_out = torch.empty((), dtype=torch.float32, device="cuda")
    for i in range(warmup + steps):
        if flush is not None:
            torch.amax(flush, dim=0, out=flush_out)
        if i >= warmup:
            ev[i - warmup][0].record(stream)
        kda.kda_fwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state, o, fs,
                    ctx, h)
        if i >= warmup:
            ev[i - warmup][1].record(stream)
        if bwd:
            kda.kda_bwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state, ctx,
                        d.do, d.dfinal_state, *grads, ws, h)
        if i >= warmup:
            ev[i - warmup][2].record(stream)
    torch.cuda.synchronize()
    f = sum(a.elapsed_time(b) for a, b, _ in ev) / steps
    b = sum(b_.elapsed_time(c) for _, b_, c in ev) / steps if bwd else None
    return f, b


def tapeless_forward(kda, p, d, inp_cpu, args, stream, flush):
    """The forward without a context (no tape written): o and the final state
    only, as inference-style callers run it."""
    prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp_cpu.cu_seqlens,
                            route=args.route)
    f, _ = _fwd_bwd_times(kda, prob, d, stream, args.steps, args.warmup, flush, bwd=False,
                          ctx_none=True)
    algo = algorithmic_fwd_bytes(p)
    gbs = algo / (f * 1e-3) / 1e9
    return {"ms_mean": round(f, 4), "token_heads_per_s": round(p.token_heads / (f * 1e-3), 1),
            "achieved_GBs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def cache_cold_forward(kda, prob, p, d, args, stream, flush):
    """The headline forward (with its tape) launched alone, each launch after
    a read of a `--flush-mb` buffer: caches and translation buffers hold
    nothing of it."""
    f, _ = _fwd_bwd_times(kda, prob, d, stream, args.steps, args.warmup, flush, bwd=False)
    gbs = algorithmic_fwd_bytes(p) / (f * 1e-3) / 1e9
    return {"ms_mean": round(f, 4), "flush_mb": args.flush_mb,
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def precision_cost(kda, p, d, inp_cpu, args, stream):
    """Forward and backward of the headline step under each precision mode:
    the automatic choice (hi/lo operands only in chunks where some channel
    keeps more than e^-2 of its state), never (single BF16 predictions), and
    every chunk.  The automatic mode's cost over "fast" is the price of its
    per-chunk check on this workload; "full" is the price of hi/lo operands
    everywhere."""
    res = {}
    for name, mode in (("auto", kda.PRECISION_AUTO), ("fast", kda.PRECISION_FAST),
                       ("full", kda.PRECISION_FULL)):
        prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp_cpu.cu_seqlens,
                                route=args.route, precision=mode)
        f, b = _fwd_bwd_times(kda, prob, d, stream, args.steps, args.warmup)
        res[name] = {"fwd_ms_mean": round(f, 4), "bwd_ms_mean": round(b, 4)}
    return res


def cold_plan_call(kda, p, d, inp_cpu, stream):
    """One forward on a length set the schedule cache has not seen (a new
    tape interval makes a new schedule: host planning, a pinned host buffer,
    a device buffer and its upload), against the same call once cached."""
    import torch
    ck = 512 + 16 * (int(time.time() * 1000) % 1000)   # a key no earlier call used
    prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp_cpu.cu_seqlens,
                            checkpoint_every=ck)
    o = torch.empty_like(d.v)
    fs = torch.empty_like(d.initial_state)
    h = stream.cuda_stream
    res = {}
    for name in ("cold", "warm"):
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t = time.perf_counter()
        a.record(stream)
        kda.kda_fwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state, o, fs,
                    None, h)
        host_ms = (time.perf_counter() - t) * 1e3
        b.record(stream)
        torch.cuda.synchronize()
        res[name] = {"host_call_ms": round(host_ms, 4), "gpu_ms": round(a.elapsed_time(b), 4)}
    return res


def other_workloads(kda, args, stream):
    """The other workloads of the suite, each drawn on the device by the same
    recipe (timing only): forward and backward means in the launch
    configuration of the automatic route, with the forward's HBM fraction.
    `packed_h12` is the packed workload's per-GPU share when its 96 heads are
    split over 8 GPUs (8 x 1024 tokens, 12 heads: 96 tasks)."""
    import torch
    import workloads
    res = {}
    items = [("fixed", workloads.workload("fixed")), ("grouped", workloads.workload("grouped")),
             ("mixed", workloads.workload("mixed")),
             ("packed_h12", (workloads.Problem([1024] * 8, 12, 12, packed=True, name="packed_h12"), 3))]
    for name, (p, seed) in items:
        d = workloads.make_inputs_on_device(p, seed, "cuda")
        prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, d.extra["cu_seqlens_cpu"])
        route = kda.kda_plan_query(prob)[0]
        f, b = _fwd_bwd_times(kda, prob, d, stream, max(args.steps // 4, 3), 2)
        gbs = algorithmic_fwd_bytes(p) / (f * 1e-3) / 1e9
        bgbs = algorithmic_bwd_bytes(p) / (b * 1e-3) / 1e9
        res[name] = {"tasks": p.N * p.Hv, "token_heads": p.token_heads,
                     "route": ROUTE_NAMES.get(route, "?"),
                     "fwd_ms_mean": round(f, 4), "fwd_frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                     "bwd_ms_mean": round(b, 4), "bwd_frac_of_hbm_peak": round(bgbs / HBM_PEAK_GBS, 4)}
        if name == "mixed":
            # the same call with the tasks dispatched in sequence order instead
            # of longest first
            probs = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens,
                                     d.extra["cu_seqlens_cpu"], schedule=kda.SCHEDULE_SEQUENCE)
            fs_, bs_ = _fwd_bwd_times(kda, probs, d, stream, max(args.steps // 4, 3), 2)
            res[name]["sequence_order"] = {"fwd_ms_mean": round(fs_, 4), "bwd_ms_mean": round(bs_, 4)}
        del d
        torch.cuda.empty_cache()
    return res


def records_context_step(kda, p, d, inp_cpu, args, stream):
    """The same training step with the per-chunk records context: the forward
    stores every chunk's records and the backward reruns no forward
    recurrence.  Timed like the main step (HIP events on the kernels' stream)."""
    import torch
    prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp_cpu.cu_seqlens,
                            route=args.route, context=kda.CONTEXT_RECORDS)
    ctx_bytes = kda.kda_fwd_ctx_bytes(prob)
    ctx = torch.empty(ctx_bytes, dtype=torch.uint8, device="cuda")
    ws = torch.empty(kda.kda_bwd_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(d.v)
    fs = torch.empty_like(d.initial_state)
    grads = (torch.empty_like(d.q), torch.empty_like(d.k), torch.empty_like(d.v),
             torch.empty_like(d.g), torch.empty_like(d.beta), torch.empty_like(d.A_log),
             torch.empty_like(d.dt_bias), torch.empty_like(d.initial_state))
    h = stream.cuda_stream

    def step():
        kda.kda_fwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                    o, fs, ctx, h)
        e1.record(stream)
        kda.kda_bwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                    ctx, d.do, d.dfinal_state, *grads, ws, h)

    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    for _ in range(max(args.warmup, 2)):
        step()
    torch.cuda.synchronize()
    fwd, bwd = [], []
    for _ in range(args.steps):
        e0.record(stream)
        step()
        e2.record(stream)
        torch.cuda.synchronize()
        fwd.append(e0.elapsed_time(e1))
        bwd.append(e1.elapsed_time(e2))
    fm, bm = sum(fwd) / len(fwd), sum(bwd) / len(bwd)
    return {"fwd_ms_mean": round(fm, 4), "bwd_ms_mean": round(bm, 4), "step_ms": round(fm + bm, 4),
            "ctx_bytes": ctx_bytes}


def inference_steps(kda, p, d, inp_cpu, args, stream):
    """kda_infer (page "flashinfer.kda.recurrent_kda") on the packed workload's
    heads, timed with HIP events on the kernels' stream.
      decode: 256 sequences x 1 token against a BF16 pool of 256 slots in a
        shuffled order (the page's defaults: log-space gate, beta as a rate);
      prefill: the packed workload's own tokens with the training settings,
        starting from its initial states rounded to BF16.
    Algorithmic bytes per token-head: q, k, v, g, o and beta as in the
    training forward, plus the BF16 state read and written once per
    (sequence, head) (2 x 32 KiB)."""
    import torch
    import workloads
    dev = torch.device("cuda")
    h = stream.cuda_stream
    res = {}
    # decode
    Nd = 256
    dp = workloads.Problem([1] * Nd, p.Hqk, p.Hv, packed=True, name="decode")
    di = workloads.make_infer_inputs(dp, 7, 1)          # token tensors; pool drawn below
    gen = torch.Generator(device=dev).manual_seed(8)
    pool = (0.1 * torch.randn((Nd, p.Hv, 128, 128), generator=gen, device=dev)).to(torch.bfloat16)
    idx_cpu = torch.randperm(Nd, generator=torch.Generator().manual_seed(9)).to(torch.int32)
    idx = idx_cpu.to(dev)
    t = [x.to(dev) for x in (di.q, di.k, di.v, di.g, di.beta)]
    o = torch.empty_like(t[2])
    cu = di.cu_seqlens.to(dev)
    prob = kda.make_infer_problem(1, Nd, p.Hqk, p.Hv, Nd, Nd, cu, di.cu_seqlens,
                                  state_indices=idx, state_indices_cpu=idx_cpu)

    # the chunked route takes only the in-kernel gate: timed with it (same sizes)
    prob_c = kda.make_infer_problem(1, Nd, p.Hqk, p.Hv, Nd, Nd, cu, di.cu_seqlens,
                                    state_indices=idx, state_indices_cpu=idx_cpu, route=1,
                                    use_gate_in_kernel=True, lower_bound=-5.0)
    A_c, dt_c = di.A_log.to(dev), di.dt_bias.to(dev)
    # the training count holds the FP32 state twice; the pool is BF16
    bf16_state = lambda prob: algorithmic_fwd_bytes(prob) - prob.N * prob.Hv * 2 * 128 * 128 * 2
    res["decode"] = _time_infer(lambda: kda.kda_infer(prob, *t, None, None, pool, o, h),
                                args, stream, Nd * p.Hv, bf16_state(dp))
    res["decode"]["workload"] = f"{Nd} sequences x 1 token, Hqk={p.Hqk}, Hv={p.Hv}, pool {Nd} slots"
    res["decode"]["kernel"] = "infer_token_kernel (the automatic route)"
    res["decode"]["chunk_route_ms_mean"] = _time_infer(
        lambda: kda.kda_infer(prob_c, *t, A_c, dt_c, pool, o, h), args, stream, Nd * p.Hv,
        bf16_state(dp))["ms_mean"]
    # prefill
    pool2 = d.initial_state.to(torch.bfloat16)
    o2 = torch.empty_like(d.v)
    prob2 = kda.make_infer_problem(p.B, p.T, p.Hqk, p.Hv, p.N, p.N, d.cu_seqlens,
                                   inp_cpu.cu_seqlens, use_gate_in_kernel=True, lower_bound=-5.0,
                                   beta_is_logit=True)

    prob2t = kda.make_infer_problem(p.B, p.T, p.Hqk, p.Hv, p.N, p.N, d.cu_seqlens,
                                    inp_cpu.cu_seqlens, use_gate_in_kernel=True, lower_bound=-5.0,
                                    beta_is_logit=True, route=2)
    args2 = (d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, pool2, o2, h)
    res["prefill"] = _time_infer(lambda: kda.kda_infer(prob2, *args2), args, stream,
                                 p.token_heads, bf16_state(p))
    res["prefill"]["workload"] = "the packed workload's tokens, training settings"
    res["prefill"]["kernel"] = "fwd_chunk_kernel<infer> (the automatic route)"
    res["prefill"]["token_route_ms_mean"] = _time_infer(
        lambda: kda.kda_infer(prob2t, *args2), args, stream, p.token_heads, bf16_state(p))["ms_mean"]
    return res


def _time_infer(fn, args, stream, token_heads, nbytes):
    import torch
    for _ in range(max(args.warmup, 2)):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_mean": round(ms, 4), "token_heads_per_s": round(token_heads / (ms * 1e-3), 1),
            "algorithmic_bytes": int(nbytes), "achieved_GBs": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


if __name__ == "__main__":
    main()
