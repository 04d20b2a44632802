"""GPU parity on the degenerate and extreme cases of the method, through the
C ABI, forward and backward against the FP64 oracle:

* the strongest decay the gate allows (the gate saturates at the lower bound,
  lambda = -5 per token, so the in-chunk factors exp(+-gc) reach e^75);
* no decay (the gate at 0: the state only accumulates);
* beta -> 1 (the delta rule recalls v exactly) and beta -> 0 (pure decay);
* zero values and zero initial state (output and final state exactly zero);
* eight value heads per q/k head;
* one long sequence (a single task) on both routes;
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
    "beta_one": (P([50, 17], 2, 2, packed=True), 203, dict(beta=20.0)),
    "beta_zero": (P([50], 1, 2, packed=True), 204, dict(beta=-20.0)),
    "zero_values_state": (P([45, 16], 1, 2, packed=True), 205, dict(v=0.0, initial_state=0.0)),
    "group8": (P([37, 64], 1, 8, packed=True), 206, {}),
    "tape_boundaries": (P([256, 257, 255, 512], 1, 1, packed=True), 207, {}),
}


@pytest.mark.parametrize("route", [1, 2], ids=["chunk", "rowsplit"])
@pytest.mark.parametrize("case", list(CASES.keys()))
def test_forward_edge(case, route):
    problem, seed, set_to = CASES[case]
    inp = _inputs(problem, seed, **set_to)
    print(f"[edge fwd] case={case} route={route} lengths={problem.lengths}", flush=True)
    o, fs, _, _ = pu.run_forward(inp, route=route, save_context=False)
    ref_o, ref_s = pu.oracle_forward(inp)
    o = o.float().cpu().numpy()
    fs = fs.cpu().numpy()
    if case == "zero_values_state":
        # nothing ever enters the state: both outputs are exactly zero
        assert np.all(o == 0.0) and np.all(fs == 0.0)
    pu.assert_close("o", o, ref_o)
    print(f"  final-state max-abs error {np.abs(fs - ref_s).max():.3g}", flush=True)
    if case == "no_decay" and route == 1:
        # Without decay nothing forgets the rounding of the chunk route's BF16
        # intra-chunk products (Akk, Kg S0^T), so its final-state error grows
        # with length (about 6e-3 at 300 tokens for |S| up to 2.5) instead of
        # staying near 5e-5 as under the configs' gates; this case is held to
        # the pages' own bar.  The FP32 row-split route meets 1e-3.
        pu.assert_close("final_state", fs, ref_s)
    else:
        pu.assert_state_close("final_state", fs, ref_s)


@pytest.mark.parametrize("route", [1, 2], ids=["fwd-chunk", "fwd-rowsplit"])
@pytest.mark.parametrize("case", list(CASES.keys()))
def test_backward_edge(case, route):
    problem, seed, set_to = CASES[case]
    inp = _inputs(problem, seed, **set_to)
    print(f"[edge bwd] case={case} fwd-route={route} lengths={problem.lengths}", flush=True)
    got = pu.run_backward(inp, route=route)
    ref = pu.oracle_backward(inp)
    pu.report_and_check(list(zip(pu.GRAD_NAMES, got, ref)))


@pytest.mark.parametrize("route", [1, 2], ids=["chunk", "rowsplit"])
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
