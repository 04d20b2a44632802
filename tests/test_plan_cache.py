"""The schedule cache past its capacity: every distinct set of sequence lengths
gets a device schedule, and the library keeps at most 1024 of them.  Beyond
that it frees the least recently used ones that no call holds, no captured
graph refers to, and no queued launch still reads.  Checked here:

* more distinct length sets than the cache holds all run;
* a length set whose schedule was evicted is planned again and gives the
  same output bit for bit;
* a backward whose forward's schedule was evicted in between still matches
  a backward run without the churn;
* a graph captured before the churn replays bit for bit after it (its
  schedule is kept for the life of the process).
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

CAPACITY = 1024       # schedules the library keeps at once
CHURN = CAPACITY + 200


class _Step:
    """Static buffers for one forward + backward on one problem."""

    def __init__(self, problem, seed):
        import gated_delta_rule_32_amd as kda
        self.kda = kda
        # the problem struct keeps raw pointers to both cu_seqlens copies
        self.inp = inp = workloads.make_inputs(problem, seed, with_adjoints=True)
        self.d = d = inp.to("cuda")
        p = problem
        self.prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp.cu_seqlens, route=1)
        self.o = torch.empty_like(d.v)
        self.fs = torch.empty_like(d.initial_state)
        self.ctx = torch.empty(kda.kda_fwd_ctx_bytes(self.prob), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(kda.kda_bwd_workspace_bytes(self.prob), dtype=torch.uint8, device="cuda")
        self.grads = [torch.empty_like(x) for x in (d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias,
                                                    d.initial_state)]

    def outputs(self):
        return [self.o, self.fs] + self.grads

    def fwd(self):
        d = self.d
        self.kda.kda_fwd(self.prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                         self.o, self.fs, self.ctx, torch.cuda.current_stream().cuda_stream)

    def bwd(self):
        d = self.d
        self.kda.kda_bwd(self.prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                         self.ctx, d.do, d.dfinal_state, *self.grads, self.ws,
                         torch.cuda.current_stream().cuda_stream)

    def run(self):
        self.fwd()
        self.bwd()


def _host(ts):
    return [t.float().cpu().numpy() for t in ts]


def _same(a, b, what):
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y, equal_nan=False), f"{what}: output {i} differs"


def test_schedule_cache_evicts_and_replans():
    import gated_delta_rule_32_amd as kda
    P = workloads.Problem
    # a captured step (its schedule is pinned) and a plain one
    cap = _Step(P([7, 40], 1, 2, packed=True), 520)
    plain = _Step(P([9, 33], 1, 1, packed=True), 521)
    for s in (cap, plain):
        s.run()
        torch.cuda.synchronize()
        s.run()
        torch.cuda.synchronize()
    ref_cap, ref_plain = _host(cap.outputs()), _host(plain.outputs())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap.run()
    torch.cuda.synchronize()

    # forward of the plain step now, its backward after the churn
    for t in plain.outputs():
        t.fill_(float("nan"))
    plain.fwd()

    # churn: one forward for each of CHURN distinct lengths (one sequence, one head)
    gen = torch.Generator(device="cuda").manual_seed(522)
    T = CHURN + 4     # the longest churn length
    q = torch.randn(1, T, 1, 128, device="cuda", generator=gen).bfloat16()
    k = torch.randn(1, T, 1, 128, device="cuda", generator=gen).bfloat16()
    v = torch.randn(1, T, 1, 128, device="cuda", generator=gen).bfloat16()
    g = torch.randn(1, T, 1, 128, device="cuda", generator=gen).bfloat16()
    beta = torch.randn(1, T, 1, device="cuda", generator=gen).bfloat16()
    A_log = torch.rand(1, device="cuda", generator=gen) * 2
    dt_bias = torch.randn(1, 128, device="cuda", generator=gen) * 0.1
    s0 = torch.randn(1, 1, 128, 128, device="cuda", generator=gen) * 0.01
    fs = torch.empty_like(s0)

    def churn_fwd(L):
        cu_cpu = torch.tensor([0, L], dtype=torch.int64)
        prob = kda.make_problem(1, L, 1, 1, 1, cu_cpu.cuda(), cu_cpu, route=1)
        o = torch.empty(1, L, 1, 128, dtype=torch.bfloat16, device="cuda")
        kda.kda_fwd(prob, q[:, :L], k[:, :L], v[:, :L], g[:, :L], beta[:, :L], A_log, dt_bias, s0,
                    o, fs, None)
        return o

    first = churn_fwd(3).float().cpu().numpy()
    print(f"[plan-cache] churning {CHURN} distinct lengths", flush=True)
    for L in range(4, CHURN + 4):
        churn_fwd(L)
    torch.cuda.synchronize()
    # length 3 was used once, before more than the capacity of newer sets:
    # its schedule has been evicted and is planned again here
    again = churn_fwd(3).float().cpu().numpy()
    assert np.array_equal(first, again)

    # the plain step's backward, its schedule evicted since its forward
    plain.bwd()
    torch.cuda.synchronize()
    _same(_host(plain.outputs()), ref_plain, "backward across eviction")

    # the graph captured before the churn
    for rep in range(2):
        for t in cap.outputs():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _same(_host(cap.outputs()), ref_cap, f"replay {rep} after the churn")
