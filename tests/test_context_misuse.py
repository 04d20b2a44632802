"""Misuse of the training context is refused before any launch.

Page "flashinfer.kda_training" (paragraph 1): inputs must not change between
the forward and the backward (tensor-version changes are rejected before the
backward), and outputs must not overlap each other, any input or the saved
context.  Paragraph 2: a context is used only on the device and stream that
created it.  The library also refuses a backward whose problem resolves to
another route than the forward that filled the context (the segment-parallel
route reads more of the context than the plain chunked one writes).
"""
from __future__ import annotations

import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

P = workloads.Problem
MISMATCH, OVERLAP = 9, 7


def _setup(problem, seed=900, route=0, ctx_route=None):
    """Inputs on the device, a forward on `route` into a context sized for
    `ctx_route` (default: the same route), and the adjoints."""
    import gated_delta_rule_32_amd as kda
    inp = workloads.make_inputs(problem, seed, with_adjoints=True)
    d = inp.to("cuda")
    p = kda.make_problem(problem.B, problem.T, problem.Hqk, problem.Hv, problem.N,
                         d.cu_seqlens, inp.cu_seqlens, route=route)
    p_size = p if ctx_route is None else kda.make_problem(
        problem.B, problem.T, problem.Hqk, problem.Hv, problem.N, d.cu_seqlens, inp.cu_seqlens,
        route=ctx_route)
    ctx = torch.empty(kda.kda_fwd_ctx_bytes(p_size), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(d.v)
    fs = torch.empty_like(d.initial_state)
    kda.kda_fwd(p, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state, o, fs, ctx)
    torch.cuda.synchronize()
    return inp, d, ctx


class _At:
    """A bare device address for the C call (never dereferenced: the call is
    refused on the host)."""

    def __init__(self, addr):
        self.addr = addr

    def data_ptr(self):
        return self.addr


def _grads(d):
    return [torch.empty_like(t) for t in (d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias,
                                         d.initial_state)]


def _bwd(kda, p, d, ctx, grads, ws, **over):
    args = dict(q=d.q, k=d.k, v=d.v, g=d.g, beta=d.beta, A_log=d.A_log, dt_bias=d.dt_bias,
                initial_state=d.initial_state, ctx=ctx, d_o=d.do, dfinal_state=d.dfinal_state)
    args.update(over)
    stream = args.pop("stream", None)
    return kda._lib.kda_bwd(
        kda.ctypes.byref(p), *(kda._ptr(args[n]) for n in ("q", "k", "v", "g", "beta", "A_log",
                                                           "dt_bias", "initial_state", "ctx")),
        args["ctx"].numel(), kda._ptr(args["d_o"]), kda._ptr(args["dfinal_state"]),
        *(kda._ptr(t) for t in grads), kda._ptr(ws), ws.numel(),
        stream if stream is not None else kda._stream_handle(d.q.device))


def test_route_mismatch_is_refused():
    """A forward forced onto the plain chunked route fills a context sized for
    the automatic (segment-parallel) route; the automatic backward must refuse
    it (it would read transfer matrices that forward never stored), and a
    backward on any route that reads only the tape accepts it."""
    import gated_delta_rule_32_amd as kda
    problem = P([2048], 1, 1, packed=False)
    p_auto = kda.make_problem(1, 2048, 1, 1, 1)
    assert kda.kda_plan_query(p_auto)[0] == kda.ROUTE_SEGMENTS
    print("[misuse] route mismatch", flush=True)
    inp, d, ctx = _setup(problem, route=kda.ROUTE_CHUNK, ctx_route=kda.ROUTE_AUTO)
    ws = torch.empty(kda.kda_bwd_workspace_bytes(p_auto), dtype=torch.uint8, device="cuda")
    grads = _grads(d)
    assert _bwd(kda, p_auto, d, ctx, grads, ws) == MISMATCH
    assert "route" in kda.kda_last_error()
    p1 = kda.make_problem(1, 2048, 1, 1, 1, route=kda.ROUTE_CHUNK)
    assert _bwd(kda, p1, d, ctx, grads, ws) == 0
    torch.cuda.synchronize()
    ref = [g.clone() for g in grads]
    p4 = kda.make_problem(1, 2048, 1, 1, 1, route=kda.ROUTE_CHUNK_SPLIT)
    assert _bwd(kda, p4, d, ctx, grads, ws) == 0
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(grads, ref))


def test_stream_and_pointer_mismatch_are_refused():
    import gated_delta_rule_32_amd as kda
    problem = P([100, 37], 1, 2, packed=True)
    print("[misuse] stream / pointers", flush=True)
    inp, d, ctx = _setup(problem)
    p = kda.make_problem(1, problem.T, 1, 2, 2, d.cu_seqlens, inp.cu_seqlens)
    ws = torch.empty(kda.kda_bwd_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    grads = _grads(d)
    other = torch.cuda.Stream()   # default priority
    assert _bwd(kda, p, d, ctx, grads, ws, stream=other.cuda_stream) == MISMATCH
    assert "stream" in kda.kda_last_error()
    q2 = d.q.clone()
    assert _bwd(kda, p, d, ctx, grads, ws, q=q2) == MISMATCH
    assert "inputs differ" in kda.kda_last_error()
    s2 = d.initial_state.clone()
    assert _bwd(kda, p, d, ctx, grads, ws, initial_state=s2) == MISMATCH
    # a context the forward never filled
    blank = torch.empty_like(ctx)
    assert _bwd(kda, p, d, blank, grads, ws) == MISMATCH
    torch.cuda.synchronize()


def test_backward_output_overlap_is_refused():
    import gated_delta_rule_32_amd as kda
    problem = P([64, 20], 1, 2, packed=True)
    print("[misuse] overlap", flush=True)
    inp, d, ctx = _setup(problem)
    p = kda.make_problem(1, problem.T, 1, 2, 2, d.cu_seqlens, inp.cu_seqlens)
    ws = torch.empty(kda.kda_bwd_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    grads = _grads(d)
    # two outputs sharing memory
    g2 = list(grads)
    g2[1] = grads[0]          # dk = dq
    assert _bwd(kda, p, d, ctx, g2, ws) == OVERLAP
    # an output overlapping an input, the context, do, or the workspace
    for i, alias in ((2, d.v), (3, d.do), (0, d.q)):
        g2 = list(grads)
        g2[i] = alias
        assert _bwd(kda, p, d, ctx, g2, ws) == OVERLAP, i
    # (only the address matters to the check: the extents come from the problem)
    g2 = list(grads)
    g2[7] = _At(ctx.data_ptr() + 64)            # dinitial_state inside the context
    assert _bwd(kda, p, d, ctx, g2, ws) == OVERLAP
    assert _bwd(kda, p, d, ctx, grads, ws, d_o=_At(ws.data_ptr() + 256)) == OVERLAP
    torch.cuda.synchronize()


def test_input_version_change_is_refused():
    """The binding records every input's tensor version at the forward and
    refuses the backward once one has changed."""
    import gated_delta_rule_32_amd as kda
    problem = P([48], 1, 1, packed=True)
    inp = workloads.make_inputs(problem, 903, with_adjoints=True)
    d = inp.to("cuda")
    print("[misuse] tensor version", flush=True)
    for name in ("q", "g", "A_log", "initial_state"):
        o, fs, ctx = kda.recurrent_kda_training_forward(
            d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
            cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens)
        getattr(d, name).mul_(1.0)   # same values, new version
        with pytest.raises(ValueError, match="tensor version"):
            kda.recurrent_kda_training_backward(ctx, d.do, d.dfinal_state)
    # unchanged inputs: accepted
    o, fs, ctx = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens)
    kda.recurrent_kda_training_backward(ctx, d.do, d.dfinal_state)
    torch.cuda.synchronize()


def test_context_reuse_on_another_stream_is_refused():
    import gated_delta_rule_32_amd as kda
    problem = P([48], 1, 1, packed=True)
    inp = workloads.make_inputs(problem, 904)
    d = inp.to("cuda")
    print("[misuse] context reuse across streams", flush=True)
    o, fs, ctx = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens)
    torch.cuda.synchronize()
    other = torch.cuda.Stream()
    with torch.cuda.stream(other):
        with pytest.raises(ValueError, match="stream"):
            kda.recurrent_kda_training_forward(
                d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
                cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens, context_out=ctx)
    torch.cuda.synchronize()
