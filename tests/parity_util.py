"""Shared helpers of the GPU parity tests: run the HIP path through the binding
and compare with the FP64 oracle at the tolerances the method fixes.

Tolerances: o and every gradient elementwise |x - ref| <= 1e-2 + 1e-2 |ref|
(page "flashinfer.kda_training", paragraph 6: validation bar), and, because
that bar is loose against these magnitudes, a Frobenius bar as well:
||x - ref|| <= 1e-2 ||ref|| + 1e-6 sqrt(n) (relative, with an absolute floor
of 1e-6 RMS so that a reference that is zero to within underflow, such as a
gate gradient through a saturated sigmoid, does not demand exact zeros); the
FP32 final state within max-abs 1e-3.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

ATOL = RTOL = 1e-2
FROB = 1e-2
FROB_ABS = 1e-6   # RMS floor of the Frobenius bar
# dA_log[h] sums dz*z over every token and channel of head h: on these inputs
# the terms' absolute sum is 300 to 2000 times the result, so an error that is
# 4e-5 of the term mass is already a 1% relative error.  Its Frobenius bar gets
# an RMS floor of 2e-3, a fifth of the pages' atol.
FROB_ABS_BY_NAME = {"dA_log": 2e-3}
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


def errors(x, ref, floor=FROB_ABS):
    """(max elementwise violation ratio, relative Frobenius error, max abs
    error, Frobenius violation ratio: error over the Frobenius bar, whose
    RMS floor is `floor`)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    x, ref = x[m], ref[m]
    diff = np.abs(x - ref)
    viol = float(np.max(diff / (ATOL + RTOL * np.abs(ref)))) if diff.size else 0.0
    nrm = float(np.linalg.norm(ref))
    err = float(np.linalg.norm(x - ref))
    frob = err / nrm if nrm > 0 else err
    fviol = err / (FROB * nrm + floor * np.sqrt(max(diff.size, 1)))
    return viol, frob, float(diff.max()) if diff.size else 0.0, fviol


def assert_close(name, x, ref):
    viol, fr, mx, fviol = errors(x, ref)
    assert viol <= 1.0, f"{name}: elementwise bar exceeded (worst ratio {viol:.3g}, max abs {mx:.3g})"
    assert fviol <= 1.0, f"{name}: Frobenius bar exceeded (relative error {fr:.3g})"
    return viol, fr, mx


def assert_state_close(name, x, ref, atol=STATE_ATOL):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    m = ~np.isnan(ref)
    mx = float(np.abs(x[m] - ref[m]).max())
    assert mx <= atol, f"{name}: max-abs error {mx:.3g} > {atol}"
    return mx


GRAD_NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias", "dinitial_state")


def run_backward(inp: workloads.Inputs, route: int = 0, ckpt: int = 0):
    """Forward with context, then the paired backward; the eight gradients as
    NumPy FP32 arrays."""
    import gated_delta_rule_32_amd as kda
    o, fs, ctx, d = run_forward(inp, route=route, ckpt=ckpt, save_context=True)
    grads = kda.recurrent_kda_training_backward(ctx, d.do, d.dfinal_state)
    torch.cuda.synchronize()
    return [g.float().cpu().numpy() for g in grads]


def report_and_check(pairs):
    """pairs: (name, got, ref) triples.  Prints every error, then asserts the
    elementwise and Frobenius bars."""
    rows = []
    for name, x, r in pairs:
        viol, fr, mx, fviol = errors(x, r, FROB_ABS_BY_NAME.get(name, FROB_ABS))
        rows.append((name, viol, fr, mx, fviol))
        print(f"  {name:16s} worst ratio {viol:.3g}  rel-frob {fr:.3g}  max-abs {mx:.3g}", flush=True)
    for name, viol, fr, mx, fviol in rows:
        assert viol <= 1.0, f"{name}: elementwise bar exceeded (worst ratio {viol:.3g}, max abs {mx:.3g})"
        assert fviol <= 1.0, f"{name}: Frobenius bar exceeded (relative error {fr:.3g})"


def task_mask_tokens(problem, tasks):
    """Boolean mask [B, T, Hv] of the token-head entries owned by `tasks`."""
    m = np.zeros((problem.B, problem.T, problem.Hv), dtype=bool)
    for (n, b, t0, L) in workloads.sequence_slices(problem):
        for (tn, th) in tasks:
            if tn == n:
                m[b, t0:t0 + L, th] = True
    return m
