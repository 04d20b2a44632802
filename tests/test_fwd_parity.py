"""GPU parity of the forward (o in BF16, final state in FP32) against the FP64
oracle, through the C ABI, on both routes.

Small problems are compared in full; the five named workloads are compared on
sampled (sequence, head) tasks that the oracle computes one by one, in the
launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

ROUTES = [1, 2, 4]  # chunked MFMA, row-split, chunked with the value columns split
ROUTE_NAMES = {1: "chunk", 2: "rowsplit", 4: "split"}


def _small_cases():
    P = workloads.Problem
    return {
        "tiny": workloads.workload("tiny"),
        "ragged": (P([1, 15, 16, 17, 33, 100], 2, 4, packed=True), 100),
        "fixed3x80": (P([80] * 3, 2, 2, packed=False), 101),
        "grouped": (P([40, 70], 2, 8, packed=True), 102),
        "single_token": (P([1], 1, 1, packed=True), 103),
    }


@pytest.mark.parametrize("route", ROUTES, ids=lambda r: ROUTE_NAMES[r])
@pytest.mark.parametrize("case", list(_small_cases().keys()))
def test_forward_small(case, route):
    problem, seed = _small_cases()[case]
    inp = workloads.make_inputs(problem, seed, with_adjoints=False)
    print(f"[fwd] case={case} route={ROUTE_NAMES[route]} lengths={problem.lengths[:8]}", flush=True)
    o, fs, _, _ = pu.run_forward(inp, route=route, save_context=False)
    ref_o, ref_s = pu.oracle_forward(inp)
    pu.assert_close("o", o.float().cpu().numpy(), ref_o)
    pu.assert_state_close("final_state", fs.cpu().numpy(), ref_s)


def _sampled_tasks(problem, k=3):
    # first, middle and last task of the sequence order, spread over heads
    N, Hv = problem.N, problem.Hv
    cand = [(0, 0), (N // 2, Hv // 2), (N - 1, Hv - 1)]
    if problem.name == "mixed":
        # include the longest sequence and a short one
        L = problem.lengths
        cand = [(int(np.argmax(L)), 1), (int(np.argmin(L)), Hv - 2), (N // 3, Hv // 3)]
    return cand[:k]


@pytest.mark.parametrize("route", ROUTES, ids=lambda r: ROUTE_NAMES[r])
@pytest.mark.parametrize("name", workloads.WORKLOADS)
def test_forward_workloads_sampled(name, route):
    inp = workloads.make_workload(name, with_adjoints=False)
    problem = inp.problem
    tasks = _sampled_tasks(problem)
    print(f"[fwd] workload={name} route={ROUTE_NAMES[route]} tasks={tasks}", flush=True)
    o, fs, _, _ = pu.run_forward(inp, route=route, save_context=True)
    ref_o, ref_s = pu.oracle_forward(inp, tasks=tasks)
    m = pu.task_mask_tokens(problem, tasks)
    o_np = o.float().cpu().numpy()
    pu.assert_close("o", o_np[m], ref_o[m])
    fs_np = fs.cpu().numpy()
    for (n, h) in tasks:
        pu.assert_state_close(f"final_state[{n},{h}]", fs_np[n, h], ref_s[n, h])
    assert np.isfinite(o_np).all() and np.isfinite(fs_np).all()


@pytest.mark.parametrize("name", ["tiny", "fixed", "grouped", "packed"])
def test_forward_workloads_full_auto(name):
    """Every task of the workload on the automatic route, with the context
    saved (as in training and the benchmark, so the fixed 2x2048 workload runs
    segment-parallel through its 256-token tape): o and every final state
    against the oracle (page "flashinfer.kda_training", paragraph 6: the full
    packed shape, all outputs)."""
    import gated_delta_rule_32_amd as kda
    inp = workloads.make_workload(name, with_adjoints=False)
    problem = inp.problem
    route = kda.kda_plan_query(kda.make_problem(problem.B, problem.T, problem.Hqk, problem.Hv,
                                                problem.N, inp.cu_seqlens, inp.cu_seqlens))[0]
    print(f"[fwd] workload={name} AUTO (route {route}), all {problem.N * problem.Hv} tasks",
          flush=True)
    o, fs, _, _ = pu.run_forward(inp, route=0, save_context=True)
    o_np = o.float().cpu().numpy()
    fs_np = fs.cpu().numpy()
    del o, fs
    ref_o, ref_s = pu.oracle_forward(inp, workers=oracle.default_workers())
    pu.report_and_check([("o", o_np, ref_o)])
    mx = pu.assert_state_close("final_state", fs_np, ref_s)
    print(f"  final-state max-abs {mx:.3g} (ratio {mx / pu.STATE_ATOL:.3g})", flush=True)


def _mixed_tasks_per_head(problem):
    """One task per value head of the mixed workload, the heads walking over
    the sequences in a stride-7 cycle of their longest-first order, so every
    sequence appears twice and the tasks sit in all three dispatch rounds."""
    order = sorted(range(problem.N), key=lambda n: -problem.lengths[n])
    return [(order[(7 * h) % problem.N], h) for h in range(problem.Hv)]


def test_forward_mixed_per_head_auto():
    inp = workloads.make_workload("mixed", with_adjoints=False)
    problem = inp.problem
    tasks = _mixed_tasks_per_head(problem)
    print(f"[fwd] workload=mixed AUTO, {len(tasks)} tasks (one per head)", flush=True)
    o, fs, _, _ = pu.run_forward(inp, route=0, save_context=True)
    o_np = o.float().cpu().numpy()
    fs_np = fs.cpu().numpy()
    del o, fs
    ref_o, ref_s = pu.oracle_forward(inp, tasks=tasks, workers=oracle.default_workers())
    m = pu.task_mask_tokens(problem, tasks)
    pu.report_and_check([("o", o_np[m], ref_o[m])])
    worst = max(pu.assert_state_close(f"final_state[{n},{h}]", fs_np[n, h], ref_s[n, h])
                for (n, h) in tasks)
    print(f"  final-state max-abs {worst:.3g} (ratio {worst / pu.STATE_ATOL:.3g})", flush=True)
    assert np.isfinite(o_np).all() and np.isfinite(fs_np).all()


@pytest.mark.parametrize("route", ROUTES, ids=lambda r: ROUTE_NAMES[r])
def test_forward_deterministic(route):
    problem, seed = _small_cases()["ragged"]
    inp = workloads.make_inputs(problem, seed, with_adjoints=False)
    o1, f1, _, _ = pu.run_forward(inp, route=route)
    o2, f2, _, _ = pu.run_forward(inp, route=route)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def _segment_cases():
    P = workloads.Problem
    return {  # (problem, seed, tape interval): several segments per sequence, tails, one-segment sequences
        "ragged_ck32": (P([1, 15, 16, 17, 33, 100, 250], 2, 4, packed=True), 110, 32),
        "fixed_ck64": (P([300] * 2, 1, 2, packed=False), 111, 64),
        "grouped_ck16": (P([40, 70], 2, 8, packed=True), 112, 16),
    }


@pytest.mark.parametrize("case", list(_segment_cases().keys()))
def test_forward_segments(case):
    """The segment-parallel route: o and the final state against the oracle,
    and its tape (states chained through the segments as S_in P + Q) against
    the plain chunked route's tape, at the FP32 state bar."""
    problem, seed, ck = _segment_cases()[case]
    inp = workloads.make_inputs(problem, seed, with_adjoints=False)
    print(f"[fwd] segments case={case} ck={ck} lengths={problem.lengths[:8]}", flush=True)
    o, fs, ctx, _ = pu.run_forward(inp, route=3, ckpt=ck, save_context=True)
    ref_o, ref_s = pu.oracle_forward(inp)
    pu.assert_close("o", o.float().cpu().numpy(), ref_o)
    pu.assert_state_close("final_state", fs.cpu().numpy(), ref_s)
    o1, f1, ctx1, _ = pu.run_forward(inp, route=1, ckpt=ck, save_context=True)
    n_ck = sum(-(-L // ck) - 1 for L in problem.lengths)
    tape_bytes = n_ck * problem.Hv * 128 * 128 * 4
    t3 = ctx.ctx[256:256 + tape_bytes].view(torch.float32).cpu().numpy()
    t1 = ctx1.ctx[256:256 + tape_bytes].view(torch.float32).cpu().numpy()
    assert np.isfinite(t3).all()
    assert np.abs(t3 - t1).max() < pu.STATE_ATOL
    assert (o.float() - o1.float()).abs().max().item() < 2e-3
    assert (fs - f1).abs().max().item() < pu.STATE_ATOL


def test_routes_agree():
    """Both routes compute the same recurrence: their outputs agree to well
    inside the tolerance."""
    problem, seed = _small_cases()["grouped"]
    inp = workloads.make_inputs(problem, seed, with_adjoints=False)
    o1, f1, _, _ = pu.run_forward(inp, route=1)
    o2, f2, _, _ = pu.run_forward(inp, route=2)
    assert (o1.float() - o2.float()).abs().max().item() < 2e-3
    assert (f1 - f2).abs().max().item() < 1e-3


def test_packed_equals_fixed_on_gpu():
    """Packed 3x64 and fixed B=3, T=64 give identical results."""
    pf = workloads.Problem([64] * 3, 2, 2, packed=False)
    inp = workloads.make_inputs(pf, 104, with_adjoints=False)
    o_f, s_f, _, _ = pu.run_forward(inp, route=2)
    pk = workloads.Problem([64] * 3, 2, 2, packed=True)
    inp_p = workloads.Inputs(pk, *(t.reshape((1, -1) + t.shape[2:]) for t in
                                   (inp.q, inp.k, inp.v, inp.g, inp.beta)),
                             inp.A_log, inp.dt_bias, inp.initial_state, pk.cu_seqlens())
    o_p, s_p, _, _ = pu.run_forward(inp_p, route=2)
    assert torch.equal(o_p.reshape(o_f.shape), o_f) and torch.equal(s_p, s_f)
