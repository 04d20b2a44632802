"""GPU parity of the backward (all eight gradients) against the FP64 oracle,
through the C ABI.

The forward saves its context (the FP32 state tape); kda_bwd rebuilds the
chunk-start states segment by segment, runs the chunk adjoint per task and
reduces dq/dk over grouped heads and dA_log/ddt_bias over tasks.  Small
problems are compared in full; the five named workloads on sampled tasks that
the oracle computes one by one (a whole q/k-head group for dq/dk, one value
head over every sequence for dA_log/ddt_bias).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

NAMES = pu.GRAD_NAMES
_run_backward = pu.run_backward
_report_and_check = pu.report_and_check


def _small_cases():
    P = workloads.Problem
    return {
        "tiny": (workloads.workload("tiny"), 0),
        "ragged": ((P([1, 15, 16, 17, 33, 100], 2, 4, packed=True), 100), 0),
        "fixed3x80": ((P([80] * 3, 2, 2, packed=False), 101), 0),
        "grouped": ((P([40, 70], 2, 8, packed=True), 102), 0),
        "single_token": ((P([1], 1, 1, packed=True), 103), 0),
        # several tape segments per sequence: the rebuild starts mid-sequence
        "segments_ck32": ((P([100, 37, 64], 1, 2, packed=True), 105), 32),
        "segments_ck16_fixed": ((P([64, 64], 2, 2, packed=False), 106), 16),
        "segments_ck16_packed": ((P([50, 16, 33], 2, 4, packed=True), 107), 16),
    }


@pytest.mark.parametrize("route", [1, 2, 3, 4], ids=["fwd-chunk", "fwd-rowsplit", "fwd-segments", "fwd-split"])
@pytest.mark.parametrize("case", list(_small_cases().keys()))
def test_backward_small(case, route):
    (problem, seed), ckpt = _small_cases()[case]
    inp = workloads.make_inputs(problem, seed, with_adjoints=True)
    print(f"[bwd] case={case} fwd-route={route} ckpt={ckpt} lengths={problem.lengths[:8]}", flush=True)
    got = _run_backward(inp, route=route, ckpt=ckpt)
    ref = pu.oracle_backward(inp)
    _report_and_check(list(zip(NAMES, got, ref)))


def _sampled(problem, spread=24):
    """Tasks the oracle runs: whole q/k-head groups (dq, dk sum over a group)
    on `spread` (sequence, q/k head) pairs taken evenly along the longest-first
    dispatch order plus the first/last (or longest/shortest) sequences, and
    one value head over every sequence (dA_log, ddt_bias sum over them)."""
    G = problem.Hv // problem.Hqk
    hq = problem.Hqk // 2
    if problem.name == "mixed":
        L = problem.lengths
        seqs = [int(np.argmax(L)), int(np.argmin(L))]
    else:
        seqs = [0, problem.N - 1] if problem.N > 1 else [0]
    pairs = {(n, hq) for n in seqs}
    order = sorted(range(problem.N), key=lambda n: -problem.lengths[n])
    qk_tasks = [(n, j) for n in order for j in range(problem.Hqk)]
    for i in np.linspace(0, len(qk_tasks) - 1, min(spread, len(qk_tasks))):
        pairs.add(qk_tasks[int(round(i))])
    pairs = sorted(pairs)
    group = [(n, j * G + g) for (n, j) in pairs for g in range(G)]
    h_par = hq * G
    every = [(n, h_par) for n in range(problem.N)]
    return pairs, h_par, sorted(set(group + every))


@pytest.mark.parametrize("name", workloads.WORKLOADS)
def test_backward_workloads_sampled(name):
    inp = workloads.make_workload(name, with_adjoints=True)
    p = inp.problem
    G = p.Hv // p.Hqk
    pairs, h_par, tasks = _sampled(p)
    print(f"[bwd] workload={name} AUTO tasks={len(tasks)} qk-groups={len(pairs)} h_par={h_par}",
          flush=True)
    got = dict(zip(NAMES, _run_backward(inp)))
    res = oracle.backward_tasks(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.A_log, inp.dt_bias,
                                inp.initial_state, inp.do, inp.dfinal_state, p.lengths, p.packed,
                                tasks, workers=oracle.default_workers())
    sl = {n: (b, t0, L) for (n, b, t0, L) in workloads.sequence_slices(p)}
    cat = {k: ([], []) for k in ("dv", "dg", "dbeta", "dinitial_state", "dq", "dk")}
    for (n, h), (dq, dk, dv, dg, dbeta, dA, ddt, dS0) in res.items():
        b, t0, L = sl[n]
        s = slice(t0, t0 + L)
        for key, ref, x in (("dv", dv, got["dv"][b, s, h]), ("dg", dg, got["dg"][b, s, h]),
                            ("dbeta", dbeta, got["dbeta"][b, s, h]),
                            ("dinitial_state", dS0, got["dinitial_state"][n, h])):
            cat[key][0].append(np.ravel(x))
            cat[key][1].append(np.ravel(ref))
    for (n, hq) in pairs:
        b, t0, L = sl[n]
        s = slice(t0, t0 + L)
        for key, idx in (("dq", 0), ("dk", 1)):
            ref = sum(res[(n, hq * G + g)][idx] for g in range(G))
            cat[key][0].append(np.ravel(got[key][b, s, hq]))
            cat[key][1].append(np.ravel(ref))
    dA_ref = sum(res[(n, h_par)][5] for n in range(p.N))
    ddt_ref = sum(res[(n, h_par)][6] for n in range(p.N))
    pairs = [(k, np.concatenate(v[0]), np.concatenate(v[1])) for k, v in cat.items()]
    pairs.append(("dA_log", np.array([got["dA_log"][h_par]]), np.array([dA_ref])))
    pairs.append(("ddt_bias", got["ddt_bias"][h_par], ddt_ref))
    _report_and_check(pairs)
    for k in NAMES:
        assert np.isfinite(got[k]).all(), f"{k} has non-finite values"


def test_backward_deterministic():
    (problem, seed), _ = _small_cases()["grouped"]
    inp = workloads.make_inputs(problem, seed, with_adjoints=True)
    g1 = _run_backward(inp, route=1)
    g2 = _run_backward(inp, route=1)
    for name, a, b in zip(NAMES, g1, g2):
        assert np.array_equal(a, b), f"{name} differs between two identical calls"
