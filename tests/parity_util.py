"""Shared helpers of the GPU parity tests: run the HIP path through the binding
and compare with the FP64 oracle at the tolerances the method fixes.

Tolerances: o and every gradient elementwise |x - ref| <= 1e-2 + 1e-2 |ref|
(page "flashinfer.kda_training", paragraph 6: validation bar), and, because
that bar is loose against these magnitudes, relative Frobenius error
||x - ref|| / ||ref|| <= 1e-2 as well; the FP32 final state within max-abs
1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

ATOL = RTOL = 1e-2
FROB = 1e-2
STATE_ATOL = 1e-3


def run_forward(inp: workloads.Inputs, route: int = 0, ckpt: int = 0, save_context=True):
    import gated_delta_rule_32_amd as kda
    d = inp.to("cuda")
    cu_cpu = inp.cu_seqlens
    o, fs, ctx = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=cu_cpu, route=route,
        checkpoint_every=ckpt, save_context=save_context)
    torch.cuda.synchronize()
    return o, fs, ctx, d


def oracle_forward(inp: workloads.Inputs, tasks=None, workers=None):
    p = inp.problem
    return oracle.forward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.A_log, inp.dt_bias,
                          inp.initial_state, p.lengths, p.packed, tasks=tasks, workers=workers)


def oracle_backward(inp: workloads.Inputs, tasks=None, workers=None):
    p = inp.problem
    return oracle.backward(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.A_log, inp.dt_bias,
                           inp.initial_state, inp.do, inp.dfinal_state, p.lengths, p.packed,
                           tasks=tasks, workers=workers)


def errors(x, ref):
    """(max elementwise violation ratio, relative Frobenius error, max abs error)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    x, ref = x[m], ref[m]
    diff = np.abs(x - ref)
    viol = float(np.max(diff / (ATOL + RTOL * np.abs(ref)))) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    frob = float(np.linalg.norm(x - ref) / nrm) if nrm > 0 else float(np.linalg.norm(x - ref))
    return viol, frob, float(diff.max()) if diff.size else 0.0


def assert_close(name, x, ref, frob=FROB):
    viol, fr, mx = errors(x, ref)
    assert viol <= 1.0, f"{name}: elementwise bar exceeded (worst ratio {viol:.3g}, max abs {mx:.3g})"
    assert fr <= frob, f"{name}: relative Frobenius error {fr:.3g} > {frob}"
    return viol, fr, mx


def assert_state_close(name, x, ref, atol=STATE_ATOL):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    mx = float(np.abs(x[m] - ref[m]).max())
    assert mx <= atol, f"{name}: max-abs error {mx:.3g} > {atol}"
    return mx


def task_mask_tokens(problem, tasks):
    """Boolean mask [B, T, Hv] of the token-head entries owned by `tasks`."""
    m = np.zeros((problem.B, problem.T, problem.Hv), dtype=bool)
    for (n, b, t0, L) in workloads.sequence_slices(problem):
        for (tn, th) in tasks:
            if tn == n:
                m[b, t0:t0 + L, th] = True
    return m
