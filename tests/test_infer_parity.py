"""GPU parity of the inference forward kda_infer (page
"flashinfer.kda.recurrent_kda": decode and prefill with the gate, beta and
norm options, on a BF16 state pool updated in place) against the FP64
inference oracle, through the C ABI.

Bar: the output and the updated pool slots (both BF16) within the pages'
validation bar |x - ref| <= 1e-2 + 1e-2 |ref| plus the Frobenius bar of
parity_util; pool slots no sequence names must come back bit for bit.  Every
case runs on the token-serial kernel and, where its per-token log-decays stay
at or above -5, on the chunked kernel as well.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import kda_infer_oracle as kio
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

P = workloads.Problem
# name: (problem, seed, pool_slots, options, generator options)
CASES = {
    # one token per sequence against a pool with spare slots, the page's defaults
    "decode_defaults": (P([1] * 48, 2, 4, packed=True), 500, 64,
                        dict(), dict()),
    # ragged prefill with the training settings (in-kernel gate, beta logits)
    "prefill_training_gate": (P([1, 15, 16, 17, 33, 100], 2, 4, packed=True), 501, 8,
                              dict(use_gate_in_kernel=True, lower_bound=-5.0, beta_is_logit=True),
                              dict(log_gate_min=None, beta_logits=True)),
    # another lower bound, and no dt_bias
    "prefill_lb3_no_dt_bias": (P([40, 7, 64], 1, 2, packed=True), 502, 3,
                               dict(use_gate_in_kernel=True, lower_bound=-3.0, no_dt_bias=True),
                               dict(log_gate_min=None)),
    # q, k used as given (near-unit draws)
    "prefill_no_norm": (P([30, 50], 2, 2, packed=True), 503, 2,
                        dict(use_qk_l2norm=False), dict(qk_std=128 ** -0.5)),
    # log-space gates down to -20 per token: no range limit on this route
    "prefill_strong_log_gate": (P([37, 80], 1, 1, packed=True), 504, 5,
                                dict(), dict(log_gate_min=-20.0)),
    # fixed layout, pool slot n for sequence n
    "fixed_identity_slots": (P([40] * 3, 1, 2, packed=False), 505, 3,
                             dict(identity_slots=True), dict()),
}


def _binding_opts(opts):
    # the page's parameter name for the norm option
    out = dict(opts)
    if "use_qk_l2norm" in out:
        out["use_qk_l2norm_in_kernel"] = out.pop("use_qk_l2norm")
    return out


# the chunked route takes only the in-kernel gate with lower_bound >= -5 (a
# log-space gate has no bound the host can check): other cases run token by
# token
TOKEN_ONLY = {c for c, v in CASES.items() if not v[3].get("use_gate_in_kernel")}
ROUTES = {"chunk": 1, "token": 2}
PARAMS = [(c, r) for c in CASES for r in ROUTES if not (r == "chunk" and c in TOKEN_ONLY)]


def _gate_gen(route):
    """Input options for the tests below that run on either route: raw gate
    inputs for the in-kernel gate on the chunked route (the only gate it
    takes), the default log-space decays token by token."""
    return dict(log_gate_min=None) if route == "chunk" else dict()


def _gate_kw(route, inp, dev):
    """The binding's and the oracle's gate arguments for _gate_gen's inputs:
    the in-kernel gate with lower bound -5 on the chunked route, none (g is
    the log-decay itself) token by token."""
    if route != "chunk":
        return dict(), dict(A_log=None, dt_bias=None)
    opts = dict(use_gate_in_kernel=True, lower_bound=-5.0)
    return (dict(A_log=inp.A_log.to(dev), dt_bias=inp.dt_bias.to(dev), **opts),
            dict(A_log=inp.A_log, dt_bias=inp.dt_bias, **opts))


def _run_case(name, route):
    import gated_delta_rule_32_amd as kda
    problem, seed, slots, opts, gen_opts = CASES[name]
    opts = dict(opts)
    no_dt = opts.pop("no_dt_bias", False)
    identity = opts.pop("identity_slots", False)
    inp = workloads.make_infer_inputs(problem, seed, slots, **gen_opts)
    idx_cpu = None if identity else inp.indices
    print(f"[infer] case={name} route={route} lengths={problem.lengths[:8]} N={problem.N} "
          f"slots={slots} options={opts}", flush=True)
    dev = torch.device("cuda")
    pool_dev = inp.pool.to(dev)
    o, pool_out = kda.recurrent_kda(
        inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev),
        A_log=inp.A_log.to(dev), dt_bias=None if no_dt else inp.dt_bias.to(dev),
        initial_state=pool_dev,
        cu_seqlens=None if inp.cu_seqlens is None else inp.cu_seqlens.to(dev),
        cu_seqlens_cpu=inp.cu_seqlens,
        ssm_state_indices=None if idx_cpu is None else idx_cpu.to(dev),
        ssm_state_indices_cpu=idx_cpu, route=ROUTES[route], output_final_state=True,
        **_binding_opts(opts))
    torch.cuda.synchronize()
    assert pool_out.data_ptr() == pool_dev.data_ptr()
    o_ref, pool_ref = kio.infer_forward(
        inp.q, inp.k, inp.v, inp.g, inp.beta, inp.A_log, None if no_dt else inp.dt_bias,
        inp.pool, problem.lengths, problem.packed,
        indices=None if idx_cpu is None else idx_cpu.tolist(), **opts)
    return problem, inp, idx_cpu, o.float().cpu().numpy(), pool_dev.float().cpu().numpy(), \
        o_ref, pool_ref


@pytest.mark.parametrize("case,route", PARAMS)
def test_infer_matches_oracle(case, route):
    problem, inp, idx_cpu, o, pool, o_ref, pool_ref = _run_case(case, route)
    named = list(range(problem.N)) if idx_cpu is None else idx_cpu.tolist()
    rest = [s for s in range(pool.shape[0]) if s not in set(named)]
    pu.report_and_check([("o", o, o_ref), ("state_pool", pool[named], pool_ref[named])])
    before = inp.pool.float().numpy()
    for s in rest:
        assert np.array_equal(pool[s], before[s]), f"pool slot {s} changed but no sequence names it"


@pytest.mark.parametrize("route", list(ROUTES.keys()))
def test_infer_training_settings_match_training_forward(route):
    """With the training settings and the pool holding the BF16-rounded
    initial states, the output matches the training forward's (both within
    the bar of the FP64 oracle, checked above); here the two GPU paths are
    compared directly on the same draws."""
    import gated_delta_rule_32_amd as kda
    problem = P([9, 40, 23], 2, 2, packed=True)
    inp = workloads.make_inputs(problem, 506, with_adjoints=False)
    s0_bf = inp.initial_state.to(torch.bfloat16)
    inp.initial_state = s0_bf.float()
    o_t, fs_t, _ctx, d = pu.run_forward(inp, save_context=False)
    pool = s0_bf.to("cuda")
    o_i, _ = kda.recurrent_kda(d.q, d.k, d.v, d.g, d.beta, A_log=d.A_log, dt_bias=d.dt_bias,
                               initial_state=pool, use_gate_in_kernel=True, lower_bound=-5.0,
                               beta_is_logit=True, cu_seqlens=d.cu_seqlens,
                               cu_seqlens_cpu=inp.cu_seqlens, route=ROUTES[route])
    torch.cuda.synchronize()
    pu.report_and_check([("o", o_i.float().cpu().numpy(), o_t.float().cpu().numpy()),
                         ("final_state", pool.float().cpu().numpy(), fs_t.cpu().numpy())])


@pytest.mark.parametrize("route,every", [("chunk", 16), ("chunk", 32), ("token", 16), ("token", 48)])
def test_infer_state_checkpoints(route, every):
    """State checkpoints (parameters state_checkpoints, checkpoint_cu_starts,
    checkpoint_every_n_tokens): row j of a sequence holds its state before
    token j*E; rows past the last start are not touched."""
    import gated_delta_rule_32_amd as kda
    problem = P([5, 16, 17, 40, 100], 1, 2, packed=True)
    inp = workloads.make_infer_inputs(problem, 507, 7, **_gate_gen(route))
    counts = [-(-L // every) for L in problem.lengths]
    starts_cpu = torch.tensor([0] + list(np.cumsum(counts)), dtype=torch.int64)
    print(f"[infer] checkpoints route={route} every={every} rows={int(starts_cpu[-1])}", flush=True)
    dev = torch.device("cuda")
    gcall, gref = _gate_kw(route, inp, dev)
    rows = int(starts_cpu[-1]) + 2
    ck = torch.full((rows, problem.Hv, 128, 128), 7.0, dtype=torch.bfloat16, device=dev)
    pool = inp.pool.to(dev)
    o, _pool, ck_out = kda.recurrent_kda(
        inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev), **gcall,
        initial_state=pool, cu_seqlens=inp.cu_seqlens.to(dev), cu_seqlens_cpu=inp.cu_seqlens,
        ssm_state_indices=inp.indices.to(dev), ssm_state_indices_cpu=inp.indices,
        state_checkpoints=ck, checkpoint_cu_starts=starts_cpu.to(dev),
        checkpoint_cu_starts_cpu=starts_cpu, checkpoint_every_n_tokens=every, route=ROUTES[route])
    torch.cuda.synchronize()
    assert ck_out.data_ptr() == ck.data_ptr()
    o_ref, pool_ref, ck_ref = kio.infer_forward(
        inp.q, inp.k, inp.v, inp.g, inp.beta, pool=inp.pool, lengths=problem.lengths, packed=True,
        indices=inp.indices.tolist(), checkpoint_every=every, **gref)
    got = ck.float().cpu().numpy()
    n_rows = int(starts_cpu[-1])
    pu.report_and_check([("o", o.float().cpu().numpy(), o_ref),
                         ("checkpoints", got[:n_rows], ck_ref)])
    # row 0 of every sequence is its initial state, exactly
    for n, s0 in enumerate(starts_cpu[:-1].tolist()):
        assert np.array_equal(got[s0], inp.pool[int(inp.indices[n])].float().numpy())
    assert (got[n_rows:] == 7.0).all()


@pytest.mark.parametrize("route", ["chunk", "token"])
def test_infer_checkpoint_rows_out_of_range_are_skipped(route):
    """The kernels read the checkpoint starts from the caller's device copy,
    which the host checks only through its mirror.  When the device copy
    names rows past the end (here every start + 1000, and one negative), no
    checkpoint row is stored, and the outputs and the pool are as without
    checkpoints."""
    import gated_delta_rule_32_amd as kda
    every = 16
    problem = P([5, 16, 40], 1, 2, packed=True)
    inp = workloads.make_infer_inputs(problem, 517, 5, **_gate_gen(route))
    counts = [-(-L // every) for L in problem.lengths]
    starts_cpu = torch.tensor([0] + list(np.cumsum(counts)), dtype=torch.int64)
    bad = starts_cpu + 1000
    bad[1] = -3
    print(f"[infer] checkpoint rows out of range route={route}", flush=True)
    dev = torch.device("cuda")
    rows = int(starts_cpu[-1])
    ck = torch.full((rows, problem.Hv, 128, 128), 7.0, dtype=torch.bfloat16, device=dev)
    args = (inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev))
    kw = dict(cu_seqlens=inp.cu_seqlens.to(dev), cu_seqlens_cpu=inp.cu_seqlens,
              ssm_state_indices=inp.indices.to(dev), ssm_state_indices_cpu=inp.indices,
              route=ROUTES[route], **_gate_kw(route, inp, dev)[0])
    pool_a, pool_b = inp.pool.to(dev), inp.pool.to(dev)
    o_a, _, _ = kda.recurrent_kda(*args, initial_state=pool_a, state_checkpoints=ck,
                                  checkpoint_cu_starts=bad.to(dev), checkpoint_cu_starts_cpu=starts_cpu,
                                  checkpoint_every_n_tokens=every, **kw)
    o_b, _ = kda.recurrent_kda(*args, initial_state=pool_b, **kw)
    torch.cuda.synchronize()
    assert (ck.float() == 7.0).all()
    assert torch.equal(o_a, o_b) and torch.equal(pool_a, pool_b)


@pytest.mark.parametrize("accepted", ["given", "omitted"])
@pytest.mark.parametrize("packed", [True, False])
def test_infer_spec_decode(accepted, packed):
    """Speculative decode (parameters num_spec_tokens, num_accepted_tokens,
    ssm_state_indices [N, 1+S]): the state starts from the slot of the last
    accepted token and the state after every token lands in that token's
    slot."""
    import gated_delta_rule_32_amd as kda
    N, S, slots = 24, 3, 128
    problem = P([1 + S] * N, 2, 4, packed=packed)
    inp = workloads.make_infer_inputs(problem, 508, slots)
    gen = torch.Generator().manual_seed(509)
    idx_cpu = torch.randperm(slots, generator=gen)[:N * (1 + S)].to(torch.int32).reshape(N, 1 + S)
    acc_cpu = torch.randint(0, 2 + S + 1, (N,), generator=gen, dtype=torch.int32)  # includes 0 and > 1+S
    print(f"[infer] spec decode packed={packed} accepted={accepted}", flush=True)
    dev = torch.device("cuda")
    pool = inp.pool.to(dev)
    o, _ = kda.recurrent_kda(
        inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev),
        initial_state=pool, cu_seqlens=None if inp.cu_seqlens is None else inp.cu_seqlens.to(dev),
        cu_seqlens_cpu=inp.cu_seqlens, ssm_state_indices=idx_cpu.to(dev),
        ssm_state_indices_cpu=idx_cpu, num_spec_tokens=S,
        num_accepted_tokens=acc_cpu.to(dev) if accepted == "given" else None)
    torch.cuda.synchronize()
    o_ref, pool_ref = kio.infer_forward(
        inp.q, inp.k, inp.v, inp.g, inp.beta, None, None, inp.pool, problem.lengths, packed,
        indices=idx_cpu.tolist(), num_spec_tokens=S,
        num_accepted=acc_cpu.tolist() if accepted == "given" else None)
    got = pool.float().cpu().numpy()
    named = idx_cpu.flatten().tolist()
    pu.report_and_check([("o", o.float().cpu().numpy(), o_ref),
                         ("token_slots", got[named], pool_ref[named])])
    before = inp.pool.float().numpy()
    for s in set(range(slots)) - set(named):
        assert np.array_equal(got[s], before[s])


@pytest.mark.parametrize("route", list(ROUTES.keys()))
def test_infer_source_pool(route):
    """Read-only source pool (parameters initial_state_source,
    initial_state_indices): sequences start from source slots (repeats
    allowed), final states land in the state pool, the source is untouched."""
    import gated_delta_rule_32_amd as kda
    problem = P([3, 40, 17, 64], 1, 2, packed=True)
    inp = workloads.make_infer_inputs(problem, 510, 6, **_gate_gen(route))
    gen = torch.Generator().manual_seed(511)
    src_cpu = (0.1 * torch.randn((3, problem.Hv, 128, 128), generator=gen)).to(torch.bfloat16)
    sidx_cpu = torch.tensor([2, 0, 2, 1], dtype=torch.int32)
    print(f"[infer] source pool route={route}", flush=True)
    dev = torch.device("cuda")
    gcall, gref = _gate_kw(route, inp, dev)
    pool, src = inp.pool.to(dev), src_cpu.to(dev)
    o, _ = kda.recurrent_kda(
        inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev), **gcall,
        initial_state=pool, cu_seqlens=inp.cu_seqlens.to(dev), cu_seqlens_cpu=inp.cu_seqlens,
        ssm_state_indices=inp.indices.to(dev), ssm_state_indices_cpu=inp.indices,
        initial_state_source=src, initial_state_indices=sidx_cpu.to(dev),
        initial_state_indices_cpu=sidx_cpu, route=ROUTES[route])
    torch.cuda.synchronize()
    o_ref, pool_ref = kio.infer_forward(
        inp.q, inp.k, inp.v, inp.g, inp.beta, pool=inp.pool, lengths=problem.lengths, packed=True,
        indices=inp.indices.tolist(), source=src_cpu, source_indices=sidx_cpu.tolist(), **gref)
    named = inp.indices.tolist()
    got = pool.float().cpu().numpy()
    pu.report_and_check([("o", o.float().cpu().numpy(), o_ref),
                         ("state_pool", got[named], pool_ref[named])])
    assert torch.equal(src.cpu(), src_cpu)
    before = inp.pool.float().numpy()
    for s in set(range(6)) - set(named):
        assert np.array_equal(got[s], before[s])


def _infer_task(inp_like, n, h, s0_task, **opts):
    """Oracle of one (sequence, head) task of an inference call started from
    s0_task [128, 128]: its output rows and final state (FP64)."""
    p = inp_like["problem"]
    sl = workloads.sequence_slices(p)[n]
    _, b, t0, L = sl
    s = slice(t0, t0 + L)
    hq = h // (p.Hv // p.Hqk)
    pick = lambda x, hh: x[b:b + 1, s, hh:hh + 1]
    o, pool = kio.infer_forward(pick(inp_like["q"], hq), pick(inp_like["k"], hq),
                                pick(inp_like["v"], h), pick(inp_like["g"], h),
                                inp_like["beta"][b:b + 1, s, h:h + 1],
                                None if inp_like["A_log"] is None else inp_like["A_log"][h:h + 1],
                                None if inp_like["dt_bias"] is None else inp_like["dt_bias"][h:h + 1],
                                s0_task[None, None], [L], True, **opts)
    return o[0, :, 0], pool[0, 0], (b, t0, L)


def test_infer_decode_bench_shape_sampled():
    """The benchmark's decode step (256 one-token sequences, 96 heads, a
    shuffled 256-slot pool) on the automatic route; sampled tasks against the
    oracle, every output finite."""
    import gated_delta_rule_32_amd as kda
    problem = P([1] * 256, 96, 96, packed=True)
    inp = workloads.make_infer_inputs(problem, 512, 256)
    print("[infer] decode at the benchmark shape", flush=True)
    dev = torch.device("cuda")
    pool = inp.pool.to(dev)
    o, _ = kda.recurrent_kda(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                             inp.beta.to(dev), initial_state=pool, cu_seqlens=inp.cu_seqlens.to(dev),
                             cu_seqlens_cpu=inp.cu_seqlens, ssm_state_indices=inp.indices.to(dev),
                             ssm_state_indices_cpu=inp.indices)
    torch.cuda.synchronize()
    o_np = o.float().cpu().numpy()
    assert np.isfinite(o_np).all()
    for (n, h) in [(0, 0), (100, 47), (255, 95)]:
        slot = int(inp.indices[n])
        ref_o, ref_s, (b, t0, L) = _infer_task(
            dict(problem=problem, q=inp.q, k=inp.k, v=inp.v, g=inp.g, beta=inp.beta, A_log=None,
                 dt_bias=None), n, h, inp.pool[slot, h])
        pu.assert_close(f"o[{n},{h}]", o_np[b, t0:t0 + L, h], ref_o)
        pu.assert_close(f"pool[{slot},{h}]", pool[slot, h].float().cpu().numpy(), ref_s)


@pytest.mark.parametrize("route", list(ROUTES.keys()))
def test_infer_prefill_packed_sampled(route):
    """The packed workload (8 x 1024 tokens, 96 heads) through kda_infer with
    the training settings, pool = initial states in BF16; sampled tasks
    against the oracle."""
    import gated_delta_rule_32_amd as kda
    inp = workloads.make_workload("packed", with_adjoints=False)
    problem = inp.problem
    s0_bf = inp.initial_state.to(torch.bfloat16)
    print(f"[infer] packed prefill route={route}", flush=True)
    d = inp.to("cuda")
    pool = s0_bf.to("cuda")
    o, _ = kda.recurrent_kda(d.q, d.k, d.v, d.g, d.beta, A_log=d.A_log, dt_bias=d.dt_bias,
                             initial_state=pool, use_gate_in_kernel=True, lower_bound=-5.0,
                             beta_is_logit=True, cu_seqlens=d.cu_seqlens,
                             cu_seqlens_cpu=inp.cu_seqlens, route=ROUTES[route])
    torch.cuda.synchronize()
    o_np = o.float().cpu().numpy()
    assert np.isfinite(o_np).all()
    for (n, h) in [(0, 0), (4, 48), (7, 95)]:
        ref_o, ref_s, (b, t0, L) = _infer_task(
            dict(problem=problem, q=inp.q, k=inp.k, v=inp.v, g=inp.g, beta=inp.beta, A_log=inp.A_log,
                 dt_bias=inp.dt_bias), n, h, s0_bf[n, h],
            use_gate_in_kernel=True, lower_bound=-5.0, beta_is_logit=True)
        pu.assert_close(f"o[{n},{h}]", o_np[b, t0:t0 + L, h], ref_o)
        pu.assert_close(f"pool[{n},{h}]", pool[n, h].float().cpu().numpy(), ref_s)


@pytest.mark.parametrize("route", list(ROUTES.keys()))
def test_infer_long_single_sequence(route):
    """One 4096-token sequence (one task per head) on either route."""
    import gated_delta_rule_32_amd as kda
    problem = P([4096], 1, 2, packed=True)
    inp = workloads.make_infer_inputs(problem, 513, 1, **_gate_gen(route))
    print(f"[infer] 4096-token sequence route={route}", flush=True)
    dev = torch.device("cuda")
    gcall, gref = _gate_kw(route, inp, dev)
    pool = inp.pool.to(dev)
    o, _ = kda.recurrent_kda(inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev),
                             inp.beta.to(dev), initial_state=pool, cu_seqlens=inp.cu_seqlens.to(dev),
                             cu_seqlens_cpu=inp.cu_seqlens, route=ROUTES[route], **gcall)
    torch.cuda.synchronize()
    o_ref, pool_ref = kio.infer_forward(inp.q, inp.k, inp.v, inp.g, inp.beta, pool=inp.pool,
                                        lengths=problem.lengths, packed=True, **gref)
    pu.report_and_check([("o", o.float().cpu().numpy(), o_ref),
                         ("state_pool", pool.float().cpu().numpy(), pool_ref)])


@pytest.mark.parametrize("route", list(ROUTES.keys()))
def test_infer_without_initial_state(route):
    """Page "flashinfer.kda.recurrent_kda", parameters initial_state (None:
    zero-initialised) and output_final_state (the final state is returned only
    when asked for): a call without a pool equals one on an explicit zero pool
    of N slots."""
    import gated_delta_rule_32_amd as kda
    problem = workloads.Problem([5, 40, 17], 2, 4, packed=True)
    inp = workloads.make_infer_inputs(problem, 77, problem.N, **_gate_gen(route))
    dev = torch.device("cuda")
    print(f"[infer] no initial state route={route}", flush=True)
    gcall, _ = _gate_kw(route, inp, dev)
    args = (inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), inp.g.to(dev), inp.beta.to(dev))
    kw = dict(cu_seqlens=inp.cu_seqlens.to(dev), cu_seqlens_cpu=inp.cu_seqlens, route=ROUTES[route],
              **gcall)
    o_a, s_a = kda.recurrent_kda(*args, **kw)
    assert s_a is None
    o_b, s_b = kda.recurrent_kda(*args, output_final_state=True, **kw)
    zero = torch.zeros((problem.N, problem.Hv, 128, 128), dtype=torch.bfloat16, device=dev)
    o_c, s_c = kda.recurrent_kda(*args, initial_state=zero, output_final_state=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_c) and torch.equal(o_b, o_c) and torch.equal(s_b, s_c)
    assert s_c.data_ptr() == zero.data_ptr()
    with pytest.raises(ValueError):
        kda.recurrent_kda(*args, ssm_state_indices=torch.arange(problem.N, dtype=torch.int32, device=dev),
                          ssm_state_indices_cpu=torch.arange(problem.N, dtype=torch.int32), **kw)
