"""kda_fwd_noalloc, the forward for callers that cannot allocate device
memory, against kda_fwd through the C ABI: the same kernels over the same
schedule, so o, the final state and the context must match bit for bit, on
two calls in a row (the second smaller, so the static scratch holds the first
call's larger schedule when it starts), on the chunked and segment-parallel
routes; its context must serve kda_bwd.  Oversized schedules are refused on
the host."""
import numpy as np
import pytest
import torch

import workloads

P = workloads.Problem


def _bufs(kda, inp, route, ckpt=0):
    d = inp.to("cuda")
    p = inp.problem
    prob = kda.make_problem(p.B, p.T, p.Hqk, p.Hv, p.N, d.cu_seqlens, inp.cu_seqlens, route=route,
                            checkpoint_every=ckpt)
    ctx = torch.zeros(kda.kda_fwd_ctx_bytes(prob), dtype=torch.uint8, device="cuda")
    return d, prob, torch.empty_like(d.v), torch.empty_like(d.initial_state), ctx


def _fwd(fn, kda, inp, route, ckpt=0):
    d, prob, o, fs, ctx = _bufs(kda, inp, route, ckpt)
    fn(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state, o, fs, ctx)
    torch.cuda.synchronize()
    return d, prob, o, fs, ctx


@pytest.mark.gpu
@pytest.mark.parametrize("route,ckpt", [(0, 0), (1, 0), (3, 64)])
def test_noalloc_forward_matches_kda_fwd(route, ckpt):
    import gated_delta_rule_32_amd as kda
    cases = [(P([1024, 777, 300, 47, 1], 2, 8, packed=True), 950),   # larger schedule first
             (P([100, 37], 1, 2, packed=True), 951)]
    for problem, seed in cases:
        print(f"[noalloc] route={route} ckpt={ckpt} lengths={problem.lengths}", flush=True)
        inp = workloads.make_inputs(problem, seed, with_adjoints=True)
        _, _, o_a, fs_a, ctx_a = _fwd(kda.kda_fwd, kda, inp, route, ckpt)
        d, prob, o_b, fs_b, ctx_b = _fwd(kda.kda_fwd_noalloc, kda, inp, route, ckpt)
        assert torch.isfinite(o_b.float()).all()
        assert torch.equal(o_a, o_b), "o differs from kda_fwd"
        assert torch.equal(fs_a, fs_b), "final state differs from kda_fwd"
        assert torch.equal(ctx_a[256:], ctx_b[256:]), "context differs from kda_fwd"
        # the no-alloc forward's context serves the backward like kda_fwd's
        grads = [torch.empty_like(t) for t in (d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias,
                                               d.initial_state)]
        ws = torch.empty(kda.kda_bwd_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
        kda.kda_bwd(prob, d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state, ctx_b,
                    d.do, d.dfinal_state, *grads, ws)
        torch.cuda.synchronize()
        for t in grads:
            assert torch.isfinite(t.float()).all()


def test_noalloc_refuses_oversized_schedule():
    """A schedule larger than the static scratch (here 2^20 tasks: 4 MiB of
    task order alone) is refused before any device work."""
    import gated_delta_rule_32_amd as kda
    B, Hv = 8192, 128
    prob = kda.make_problem(B, 1, Hv, Hv, B)
    base = 1 << 40
    tensors = [base + i * (1 << 37) for i in range(11)]   # spans up to 68 GB apart
    st = kda._lib.kda_fwd_noalloc(kda.ctypes.byref(prob), *tensors[:10], None, 0, None)
    assert st == 10, kda.kda_last_error()
    assert "static scratch" in kda.kda_last_error()
