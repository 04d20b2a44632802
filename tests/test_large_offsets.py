"""Maximum sizes: element offsets past 2^31.

The kernels address a sequence's rows as a 64-bit per-sequence base plus a
32-bit offset inside the sequence, and the host refuses a sequence whose span
(L x Hv x 128 elements) reaches 2^31.  Here two packed sequences of 8192
tokens with 1100 heads each span 1.15e9 elements (inside that limit) while
the whole tensors span 2.31e9 (past it): the second sequence's rows, and the
records, tape and states of its last heads, are reachable only through the
64-bit bases.  Forward (o, final state) and backward (all eight gradients) of
tasks at both ends are compared with the FP64 oracle, each task on its own
(its inputs copied back from the device).  The forward runs again on the
column-split route (whose kernel addresses rows the same way) and is checked
at the same tasks.

Inputs are drawn on the device from a seeded generator with the workloads'
distributions (drawing 4.6 GB tensors on the host would take minutes); the
oracle's inputs are those same values, copied back.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

P = workloads.Problem
L, H = 8192, 1100


def _task_inputs(d, n, h):
    """The (sequence n, head h) task of `d` as a one-sequence, one-head CPU problem."""
    t0 = n * L
    sl = slice(t0, t0 + L)
    cpu = lambda x: x.detach().to("cpu")
    q = cpu(d.q[:, sl, h:h + 1])
    k = cpu(d.k[:, sl, h:h + 1])
    v = cpu(d.v[:, sl, h:h + 1])
    g = cpu(d.g[:, sl, h:h + 1])
    beta = cpu(d.beta[:, sl, h:h + 1])
    prob = P([L], 1, 1, packed=True)
    return workloads.Inputs(prob, q, k, v, g, beta, cpu(d.A_log[h:h + 1]), cpu(d.dt_bias[h:h + 1]),
                            cpu(d.initial_state[n:n + 1, h:h + 1]), prob.cu_seqlens(),
                            cpu(d.do[:, sl, h:h + 1]), cpu(d.dfinal_state[n:n + 1, h:h + 1]))


def test_offsets_past_2_31():
    import gated_delta_rule_32_amd as kda
    problem = P([L, L], H, H, packed=True, name="large")
    assert L * H * 128 < 2 ** 31 < problem.T * H * 128
    print(f"[large] 2 x {L} tokens x {H} heads: {problem.T * H * 128 / 2**31:.2f} x 2^31 elements",
          flush=True)
    d = workloads.make_inputs_on_device(problem, 2027, "cuda", with_adjoints=True)
    o, fs, ctx = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=d.extra["cu_seqlens_cpu"])
    grads = kda.recurrent_kda_training_backward(ctx, d.do, d.dfinal_state)
    o4, fs4, _ = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=d.extra["cu_seqlens_cpu"], route=kda.ROUTE_CHUNK_SPLIT)
    torch.cuda.synchronize()
    print("  device work done", flush=True)
    for (n, h) in ((1, H - 1), (0, 3)):
        inp = _task_inputs(d, n, h)
        sl = slice(n * L, n * L + L)
        ref_o, ref_s = pu.oracle_forward(inp)
        got_o = o[:, sl, h:h + 1].float().cpu().numpy()
        pu.report_and_check([("o", got_o, ref_o)])
        pu.assert_state_close("final_state", fs[n:n + 1, h:h + 1].cpu().numpy(), ref_s)
        pu.report_and_check([("o (column split)", o4[:, sl, h:h + 1].float().cpu().numpy(), ref_o)])
        pu.assert_state_close("final_state (column split)", fs4[n:n + 1, h:h + 1].cpu().numpy(), ref_s)
        ref_g = pu.oracle_backward(inp)
        dq, dk, dv, dg, dbeta, dA, ddt, dS0 = grads
        got = [dq[:, sl, h:h + 1], dk[:, sl, h:h + 1], dv[:, sl, h:h + 1], dg[:, sl, h:h + 1],
               dbeta[:, sl, h:h + 1], None, None, dS0[n:n + 1, h:h + 1]]
        pairs = [(name, x.float().cpu().numpy(), r)
                 for name, x, r in zip(pu.GRAD_NAMES, got, ref_g) if x is not None]
        print(f"  task (n={n}, h={h})", flush=True)
        pu.report_and_check(pairs)
        assert np.isfinite(got_o).all()
    del o, fs, ctx, grads, d, o4, fs4
    torch.cuda.empty_cache()
