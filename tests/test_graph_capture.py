"""kda_fwd and kda_bwd recorded into a HIP graph (torch.cuda.CUDAGraph) and
replayed: every replay must reproduce the eager results bit for bit (the
kernels are deterministic), with eager work and synchronisations between the
replays, and every replay's o, final state and eight gradients must meet the
method's bars against the FP64 oracle.  A call under capture whose schedule is not cached yet must fail on
the host with KDA_ERR_CAPTURE and enqueue nothing.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

P = workloads.Problem
CASES = {  # (problem, seed, context kind, route, tape interval)
    "ragged_tape": (P([1, 15, 16, 17, 33, 100, 300], 2, 4, packed=True), 400, 0, 1, 0),
    "ragged_records": (P([5, 64, 250], 1, 2, packed=True), 401, 1, 1, 0),
    "fixed_tape": (P([96] * 2, 2, 2, packed=False), 402, 0, 1, 0),
    # the segment-parallel route: P/Q, chain and rerun launches, and the
    # segmented adjoint's two passes and reverse chain
    "segments_tape": (P([300, 47, 200], 1, 2, packed=True), 403, 0, 3, 64),
}


class _Step:
    """Static buffers for one forward + backward, so that the captured
    launches keep valid pointers."""

    def __init__(self, inp, context, route=1, ckpt=0):
        import gated_delta_rule_32_amd as kda
        self.kda = kda
        self.d = d = inp.to("cuda")
        p = inp.problem
        self.prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp.cu_seqlens,
                                     route=route, checkpoint_every=ckpt, context=context)
        self.o = torch.empty_like(d.v)
        self.fs = torch.empty_like(d.initial_state)
        self.ctx = torch.empty(kda.kda_fwd_ctx_bytes(self.prob), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(kda.kda_bwd_workspace_bytes(self.prob), dtype=torch.uint8, device="cuda")
        self.grads = [torch.empty_like(x) for x in (d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias,
                                                    d.initial_state)]

    def outputs(self):
        return [self.o, self.fs] + self.grads

    def run(self):
        d, kda = self.d, self.kda
        h = torch.cuda.current_stream().cuda_stream
        kda.kda_fwd(self.prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                    self.o, self.fs, self.ctx, h)
        kda.kda_bwd(self.prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                    self.ctx, d.do, d.dfinal_state, *self.grads, self.ws, h)


def _host(ts):
    return [t.float().cpu().numpy() for t in ts]


@pytest.mark.parametrize("case", list(CASES.keys()))
def test_captured_step_replays_match_eager(case):
    problem, seed, context, route, ckpt = CASES[case]
    inp = workloads.make_inputs(problem, seed, with_adjoints=True)
    print(f"[graph] case={case} lengths={problem.lengths}", flush=True)
    step = _Step(inp, context, route, ckpt)
    # two eager calls: the first makes and uploads the schedule, the second
    # (after the device finished) observes the upload as complete
    step.run()
    torch.cuda.synchronize()
    step.run()
    torch.cuda.synchronize()
    eager = _host(step.outputs())

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step.run()
    torch.cuda.synchronize()
    ref_o, ref_s = pu.oracle_forward(inp)
    ref_g = pu.oracle_backward(inp)
    for rep in range(4):
        # eager work between replays: clobber every output, then replay
        for t in step.outputs():
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _host(step.outputs())
        for i, (a, b) in enumerate(zip(got, eager)):
            assert np.array_equal(a, b), f"replay {rep}: output {i} differs from the eager result"
        print(f"  replay {rep} against the oracle", flush=True)
        pu.report_and_check([("o", got[0], ref_o)] + list(zip(pu.GRAD_NAMES, got[2:], ref_g)))
        pu.assert_state_close(f"replay {rep} final_state", got[1], ref_s)
    # an eager call after the replays still matches as well
    step.run()
    torch.cuda.synchronize()
    for a, b in zip(_host(step.outputs()), eager):
        assert np.array_equal(a, b)


def test_capture_without_cached_schedule_is_refused():
    import gated_delta_rule_32_amd as kda
    inp = workloads.make_inputs(P([7, 41, 123], 1, 2, packed=True), 403, with_adjoints=True)
    step = _Step(inp, kda.CONTEXT_TAPE)
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(kda.KdaValueError) as ei:
        with torch.cuda.graph(graph):
            step.run()
    assert ei.value.status == kda.KDA_ERR_CAPTURE
    torch.cuda.synchronize()
    # outside capture the same call works and caches the schedule
    step.run()
    torch.cuda.synchronize()
    assert np.isfinite(step.o.float().cpu().numpy()).all()


@pytest.mark.parametrize("route", [1, 2])
def test_captured_inference_replays_match_eager(route):
    """kda_infer under capture: every replay, started from the same pool
    contents, must reproduce the eager call bit for bit (the pool is updated
    in place, so it is restored before each replay)."""
    import gated_delta_rule_32_amd as kda
    problem = P([1, 9, 33, 16], 1, 2, packed=True)
    # the chunked route takes only the in-kernel gate (raw g, lower bound -5)
    chunk = route == 1
    inp = workloads.make_infer_inputs(problem, 404 + route, 6,
                                      **(dict(log_gate_min=None) if chunk else {}))
    print(f"[graph] inference route={route}", flush=True)
    dev = torch.device("cuda")
    t = [x.to(dev) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta)]
    cu, idx = inp.cu_seqlens.to(dev), inp.indices.to(dev)
    pool0 = inp.pool.to(dev)
    pool = pool0.clone()
    o = torch.empty_like(t[2])
    prob = kda.make_infer_problem(1, problem.T, problem.Hqk, problem.Hv, problem.N, 6, cu,
                                  inp.cu_seqlens, state_indices=idx, state_indices_cpu=inp.indices,
                                  route=route, use_gate_in_kernel=chunk,
                                  lower_bound=-5.0 if chunk else None)
    A_log = inp.A_log.to(dev) if chunk else None
    dt_bias = inp.dt_bias.to(dev) if chunk else None

    def run():
        kda.kda_infer(prob, *t, A_log, dt_bias, pool, o, torch.cuda.current_stream().cuda_stream)
    for _ in range(2):                      # make the schedule, then see it settled
        pool.copy_(pool0)
        run()
        torch.cuda.synchronize()
    eager_o, eager_pool = o.clone(), pool.clone()
    graph = torch.cuda.CUDAGraph()
    pool.copy_(pool0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        run()
    torch.cuda.synchronize()
    for rep in range(3):
        pool.copy_(pool0)
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager_o), f"replay {rep}: output differs"
        assert torch.equal(pool, eager_pool), f"replay {rep}: pool differs"
