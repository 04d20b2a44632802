"""GPU parity of the records context (the forward stores the chunks'
records, the backward reruns no forward recurrence), through the C ABI, with
a start state per chunk and, with more than 256 tasks, pair records.  The records are the same arithmetic as the tape context's rebuilt ones
on the same (plain chunked) route, so o, the final state and all eight
gradients must equal that tape context's bit for bit; they are also checked
against the FP64 oracle.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import parity_util as pu

pytestmark = pytest.mark.gpu


def _run(inp, context):
    import gated_delta_rule_32_amd as kda
    d = inp.to("cuda")
    o, fs, ctx = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens, context=context,
        route=kda.ROUTE_CHUNK)
    grads = kda.recurrent_kda_training_backward(ctx, d.do, d.dfinal_state)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), fs.cpu().numpy(), [g.float().cpu().numpy() for g in grads]


P = workloads.Problem
CASES = {
    "ragged": (P([1, 15, 16, 17, 33, 100], 2, 4, packed=True), 300),
    "fixed3x80": (P([80] * 3, 2, 2, packed=False), 301),
    "long_segments": (P([600, 257], 1, 2, packed=True), 302),
    # 258 tasks: pair records (the start state of every other chunk) in both
    # contexts, odd-length sequences included
    "pair_records": (P([300, 37] + [40] * 127, 1, 2, packed=True), 303),
}


@pytest.mark.parametrize("case", list(CASES.keys()))
def test_records_context_matches_tape_and_oracle(case):
    import gated_delta_rule_32_amd as kda
    problem, seed = CASES[case]
    inp = workloads.make_inputs(problem, seed, with_adjoints=True)
    print(f"[records] case={case} lengths={problem.lengths}", flush=True)
    o_r, fs_r, g_r = _run(inp, kda.CONTEXT_RECORDS)
    o_t, fs_t, g_t = _run(inp, kda.CONTEXT_TAPE)
    assert np.array_equal(o_r, o_t) and np.array_equal(fs_r, fs_t)
    for name, a, b in zip(pu.GRAD_NAMES, g_r, g_t):
        assert np.array_equal(a, b), f"{name}: records and tape contexts differ"
    ref = pu.oracle_backward(inp)
    pu.report_and_check(list(zip(pu.GRAD_NAMES, g_r, ref)))
