"""GPU parity on the degenerate and extreme cases of the method, through the
C ABI, forward and backward against the FP64 oracle:

* the strongest decay the gate allows (the gate saturates at the lower bound,
  lambda = -5 per token, so the in-chunk factors exp(+-gc) reach e^75);
* no decay (the gate at 0: the state only accumulates) and weak decay
  (alpha = 0.99 per token) over 300, 1024 and 4096 tokens: nothing forgets the
  rounding of the chunk form's state predictions, so these hold the chunked
  route's precise chunks to the FP32 state bar;
* beta -> 1 (the delta rule recalls v exactly) and beta -> 0 (pure decay);
* zero values and zero initial state (output and final state exactly zero);
* eight value heads per q/k head;
* one long sequence (a single task) on the chunked, row-split and column-split routes;
* sequence lengths on and around the tape interval.

Inputs are the seeded draws of the workload generator with the named tensors
then set to the extreme value.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

P = workloads.Problem


def _inputs(problem, seed, **set_to):
    inp = workloads.make_inputs(problem, seed, with_adjoints=True)
    for name, value in set_to.items():
        t = getattr(inp, name)
        t.fill_(value)
    return inp


CASES = {
    # z = e^2 (8 + dt) ~ 59: sigmoid(z) = 1 to FP32, lambda = -5 per token
    "max_decay": (P([40, 33], 2, 2, packed=True), 201, dict(g=8.0, A_log=2.0)),
    # z = e^2 (-30 + dt) ~ -222: sigmoid(z) = 0 to FP32, no decay over 300 tokens
    "no_decay": (P([300], 1, 2, packed=True), 202, dict(g=-30.0, A_log=2.0)),
    # alpha = exp(-5 sigmoid(g)) with A_log = dt_bias = 0: g = -6.2 gives 0.99
    "weak_decay_1024": (P([1024], 1, 2, packed=True), 209, dict(g=-6.2, A_log=0.0, dt_bias=0.0)),
    "no_decay_1024": (P([1024], 1, 2, packed=True), 210, dict(g=-30.0, A_log=2.0)),
    "weak_decay_4096": (P([4096], 1, 1, packed=True), 211, dict(g=-6.2, A_log=0.0, dt_bias=0.0)),
    "no_decay_4096": (P([4096], 1, 1, packed=True), 212, dict(g=-30.0, A_log=2.0)),
    "beta_one": (P([50, 17], 2, 2, packed=True), 203, dict(beta=20.0)),
    "beta_zero": (P([50], 1, 2, packed=True), 204, dict(beta=-20.0)),
    "zero_values_state": (P([45, 16], 1, 2, packed=True), 205, dict(v=0.0, initial_state=0.0)),
    "group8": (P([37, 64], 1, 8, packed=True), 206, {}),
    "tape_boundaries": (P([256, 257, 255, 512], 1, 1, packed=True), 207, {}),
}


# route 3: the segment-parallel chunked route through a 64-token tape (it needs
# the context), whose P and Q runs take the same precise chunks
@pytest.mark.parametrize("route", [1, 2, 3, 4], ids=["chunk", "rowsplit", "segments", "split"])
@pytest.mark.parametrize("case", list(CASES.keys()))
def test_forward_edge(case, route):
    problem, seed, set_to = CASES[case]
    inp = _inputs(problem, seed, **set_to)
    print(f"[edge fwd] case={case} route={route} lengths={problem.lengths}", flush=True)
    ck = 64 if route == 3 else 0
    o, fs, _, _ = pu.run_forward(inp, route=route, ckpt=ck, save_context=route == 3)
    ref_o, ref_s = pu.oracle_forward(inp)
    o = o.float().cpu().numpy()
    fs = fs.cpu().numpy()
    if case == "zero_values_state":
        # nothing ever enters the state: both outputs are exactly zero
        assert np.all(o == 0.0) and np.all(fs == 0.0)
    pu.assert_close("o", o, ref_o)
    mx = pu.assert_state_close("final_state", fs, ref_s)
    print(f"  final-state max-abs error {mx:.3g}", flush=True)


@pytest.mark.parametrize("case", ["no_decay", "no_decay_1024"])
def test_fast_precision_drifts_without_decay(case):
    """What the precise chunks are for: forced off (KDA_PRECISION_FAST), the
    chunked route's final state drifts past the 1e-3 bar when nothing decays,
    while every chunk forced precise (FULL) matches the automatic choice's
    accuracy."""
    import gated_delta_rule_32_amd as kda
    problem, seed, set_to = CASES[case]
    inp = _inputs(problem, seed, **set_to)
    d = inp.to("cuda")
    ref_o, ref_s = pu.oracle_forward(inp)
    errs = {}
    for prec in (kda.PRECISION_FAST, kda.PRECISION_FULL, kda.PRECISION_AUTO):
        o, fs, _ = kda.recurrent_kda_training_forward(
            d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
            cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens, route=kda.ROUTE_CHUNK,
            save_context=False, precision=prec)
        torch.cuda.synchronize()
        pu.assert_close("o", o.float().cpu().numpy(), ref_o)
        errs[prec] = float(np.abs(fs.cpu().numpy() - ref_s).max())
    print(f"  final-state max-abs: fast {errs[kda.PRECISION_FAST]:.3g} "
          f"full {errs[kda.PRECISION_FULL]:.3g} auto {errs[kda.PRECISION_AUTO]:.3g}", flush=True)
    assert errs[kda.PRECISION_FAST] > pu.STATE_ATOL
    assert errs[kda.PRECISION_FULL] <= pu.STATE_ATOL and errs[kda.PRECISION_AUTO] <= pu.STATE_ATOL


@pytest.mark.parametrize("name", ["packed", "mixed"])
def test_full_precision_on_workload(name):
    """Every chunk forced precise on a benchmark workload (sampled tasks):
    the precise path itself at full size, not only where weak decay picks it."""
    import gated_delta_rule_32_amd as kda
    inp = workloads.make_workload(name, with_adjoints=False)
    problem = inp.problem
    d = inp.to("cuda")
    tasks = [(0, 0), (problem.N // 2, problem.Hv // 2), (problem.N - 1, problem.Hv - 1)]
    print(f"[edge] precision FULL on {name}, tasks {tasks}", flush=True)
    o, fs, _ = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens, save_context=True,
        precision=kda.PRECISION_FULL)
    torch.cuda.synchronize()
    ref_o, ref_s = pu.oracle_forward(inp, tasks=tasks)
    m = pu.task_mask_tokens(problem, tasks)
    pu.report_and_check([("o", o.float().cpu().numpy()[m], ref_o[m])])
    fs = fs.cpu().numpy()
    for (n, h) in tasks:
        pu.assert_state_close(f"final_state[{n},{h}]", fs[n, h], ref_s[n, h])


# after a route-3 forward the backward is the segment-parallel one (the dS
# chain through each 64-token segment's affine map)
@pytest.mark.parametrize("route", [1, 2, 3, 4], ids=["fwd-chunk", "fwd-rowsplit", "fwd-segments", "fwd-split"])
@pytest.mark.parametrize("case", list(CASES.keys()))
def test_backward_edge(case, route):
    problem, seed, set_to = CASES[case]
    inp = _inputs(problem, seed, **set_to)
    print(f"[edge bwd] case={case} fwd-route={route} lengths={problem.lengths}", flush=True)
    got = pu.run_backward(inp, route=route, ckpt=64 if route == 3 else 0)
    ref = pu.oracle_backward(inp)
    pu.report_and_check(list(zip(pu.GRAD_NAMES, got, ref)))


@pytest.mark.parametrize("case", ["no_decay", "weak_decay"])
def test_backward_pair_records(case):
    """More than 256 tasks (65 sequences of 1024 tokens x 4 value heads), so
    the rebuild stores the start state of every other chunk only and the
    adjoint forms the odd chunks' start states from their pairs; without
    decay, and with weak decay, nothing forgets their rounding.  The
    gradients of every value head of two sequences against the oracle (dq and
    dk are then complete; dA_log and ddt_bias sum over every sequence and are
    not compared here)."""
    set_to = dict(g=-30.0, A_log=2.0) if case == "no_decay" else dict(g=-6.2, A_log=0.0, dt_bias=0.0)
    problem = P([1024] * 65, 1, 4, packed=True)
    inp = _inputs(problem, 213, **set_to)
    print(f"[edge bwd] pair records, {case}, {problem.N * problem.Hv} tasks", flush=True)
    got = pu.run_backward(inp, route=1)
    tasks = [(n, h) for n in (0, 64) for h in range(problem.Hv)]
    ref = pu.oracle_backward(inp, tasks=tasks)
    m = pu.task_mask_tokens(problem, tasks)            # [B, T, Hv]
    mt = m.any(axis=2)                                 # [B, T]
    pairs = [("dq", got[0][mt], ref[0][mt]), ("dk", got[1][mt], ref[1][mt]),
             ("dv", got[2][m], ref[2][m]), ("dg", got[3][m], ref[3][m]),
             ("dbeta", got[4][m], ref[4][m])]
    for (n, h) in tasks:
        pairs.append((f"dinitial_state[{n},{h}]", got[7][n, h], ref[7][n, h]))
    pu.report_and_check(pairs)


@pytest.mark.parametrize("route", [1, 2, 4], ids=["chunk", "rowsplit", "split"])
def test_long_single_sequence(route):
    """One 4096-token sequence and one head: a single task, 256 chunks in
    sequence on the chunked route, 4096 steps on the row-split route."""
    problem = P([4096], 1, 1, packed=True)
    inp = workloads.make_inputs(problem, 208, with_adjoints=True)
    print(f"[edge] long single sequence, route {route}", flush=True)
    o, fs, _, _ = pu.run_forward(inp, route=route, save_context=False)
    ref_o, ref_s = pu.oracle_forward(inp)
    pu.assert_close("o", o.float().cpu().numpy(), ref_o)
    pu.assert_state_close("final_state", fs.cpu().numpy(), ref_s)
    got = pu.run_backward(inp, route=route)
    ref = pu.oracle_backward(inp)
    pu.report_and_check(list(zip(pu.GRAD_NAMES, got, ref)))


@pytest.mark.parametrize("route", [1, 3, 4], ids=["chunk", "segments", "split"])
def test_forward_huge_values(route):
    """Values of order 1e5: U leaves FP16's range, so the plain chunks' FP16
    state update scales U (and the state with it) by a power of two for the
    product.  o and the final state are linear in (v, initial state), and v
    dominates here, so both are compared after dividing by the value scale
    2e5: the pages' bar (atol = rtol = 1e-2) on the scaled quantities, and the
    scaled final state within 1e-3 (FP32 resolves about 0.01 at 1e5)."""
    problem = P([64, 37], 1, 2, packed=True)
    inp = workloads.make_inputs(problem, 213, with_adjoints=False)
    inp.v = (inp.v.float() * 2.0e5).to(torch.bfloat16)
    print(f"[edge fwd] huge values route={route}", flush=True)
    o, fs, _, _ = pu.run_forward(inp, route=route, ckpt=32 if route == 3 else 0,
                                 save_context=route == 3)
    ref_o, ref_s = pu.oracle_forward(inp)
    o = o.float().cpu().numpy()
    fs = fs.cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(fs).all()
    print(f"  max |o| {np.abs(ref_o).max():.3g}, max |S| {np.abs(ref_s).max():.3g}", flush=True)
    sc = 2.0e5
    pu.report_and_check([("o", o / sc, ref_o / sc)])
    pu.assert_state_close("final_state / 2e5", fs / sc, ref_s / sc)
