"""Pins of the FP64 oracle against facts that do not come from the oracle itself.

Each test cites the page passage it follows (FlashInfer KDA documentation).
The recurrence the oracle evaluates is: decay the state per key channel,
compute the delta-rule error from the decayed state, update, then read out.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import kda_oracle as ko

HERE = os.path.dirname(os.path.abspath(__file__))
rng_seed = 1234


def _rng(seed=rng_seed):
    return np.random.default_rng(seed)


def _task(rng, L, d, beta_scale=1.0):
    q, k, v, g = (rng.standard_normal((L, d)) for _ in range(4))
    beta = beta_scale * rng.standard_normal(L)
    A = float(rng.uniform(0, 2))
    dtb = 0.1 * rng.standard_normal(d)
    S0 = 0.01 * rng.standard_normal((d, d))
    return q, k, v, g, beta, A, dtb, S0


# ---------------------------------------------------------------------------
# hand-worked example (tests/golden/hand_worked_d2.json)
# ---------------------------------------------------------------------------
def test_hand_worked_two_tokens():
    """Two tokens at K=V=2 worked by hand: pins the update order (decay, then
    the delta error from the decayed state, then the read-out from the updated
    state), the value-first state layout and beta's sigmoid ("recurrent_kda_
    backward" description; training-forward parameter initial_state)."""
    fx = json.load(open(os.path.join(HERE, "golden", "hand_worked_d2.json")))
    a = {k: np.asarray(v, dtype=np.float64) for k, v in fx.items()
         if k not in ("about", "derivation")}
    o, S = ko.forward_task(a["q"], a["k"], a["v"], a["g"], a["beta"], float(a["A_log"]),
                           a["dt_bias"], a["S0"], scale=float(a["scale"]))
    tol = float(a["tolerance"])
    np.testing.assert_allclose(o, a["expected_o"], rtol=0, atol=tol)
    np.testing.assert_allclose(S, a["expected_final_state"], rtol=0, atol=tol)


# ---------------------------------------------------------------------------
# prologue against library routines
# ---------------------------------------------------------------------------
def test_prologue_matches_library_routines():
    """L2 norm with eps 1e-6, gate exp(lb*sigmoid(exp(A_log)(g+dt_bias))) and
    beta = sigmoid(logit) ("recurrent_kda_backward" description) against
    torch.nn.functional.normalize, scipy.special.expit and torch.exp."""
    rng = _rng()
    q, k, v, g, beta, A, dtb, S0 = _task(rng, 9, 128)
    qn, kn, lam, alpha, b, z = ko.prologue(q, k, g, beta, A, dtb)
    tq = torch.nn.functional.normalize(torch.from_numpy(q), dim=-1).numpy()
    tk = torch.nn.functional.normalize(torch.from_numpy(k), dim=-1).numpy()
    # normalize uses x/max(|x|, 1e-12); the eps inside the root differs by
    # eps/|x|^2 ~ 1e-8 relative for 128-dim N(0,1) rows.
    np.testing.assert_allclose(qn, tq, rtol=1e-7, atol=0)
    np.testing.assert_allclose(kn, tk, rtol=1e-7, atol=0)
    gate = torch.exp(-5.0 * torch.sigmoid(math.exp(A) * (torch.from_numpy(g)
                                                         + torch.from_numpy(dtb))))
    np.testing.assert_allclose(alpha, gate.numpy(), rtol=1e-13, atol=0)
    np.testing.assert_allclose(lam, np.log(gate.numpy()), rtol=1e-12, atol=0)
    np.testing.assert_allclose(b, scipy.special.expit(beta), rtol=1e-14, atol=0)
    assert np.all(lam < 0) and np.all(lam > -5)


# ---------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------
def test_single_token_from_zero_state():
    """From S0 = 0 one update gives S1 = beta v k^T, so o1 = s beta v (k.q)."""
    rng = _rng(1)
    q, k, v, g, beta, A, dtb, S0 = _task(rng, 1, 128)
    o, S = ko.forward_task(q, k, v, g, beta, A, dtb, np.zeros((128, 128)))
    kn = torch.nn.functional.normalize(torch.from_numpy(k[0]), dim=0).numpy()
    qn = torch.nn.functional.normalize(torch.from_numpy(q[0]), dim=0).numpy()
    b = scipy.special.expit(beta[0])
    np.testing.assert_allclose(S, b * np.outer(v[0], kn), rtol=1e-7, atol=1e-14)
    np.testing.assert_allclose(o[0], ko.SCALE * b * v[0] * float(kn @ qn), rtol=1e-7,
                               atol=1e-14)


def test_beta_one_makes_state_recall_value():
    """With beta = 1 (logit 40) the delta rule makes S_t k_t = v_t for a unit
    key: S_t k = P k + (v - P k)(k.k) = v when |k| = 1."""
    rng = _rng(2)
    L, d = 20, 128
    q, k, v, g, beta, A, dtb, S0 = _task(rng, L, d)
    beta[:] = 40.0
    qn, kn, lam, alpha, b, z = ko.prologue(q, k, g, beta, A, dtb)
    _, _, states = ko.recurrence(qn, kn, v, alpha, b, S0, keep_states=True)
    for t in range(L):
        # |kn|^2 = 1 - eps/(|k|^2+eps): the residual is that small
        np.testing.assert_allclose(states[t + 1] @ kn[t], v[t], rtol=0, atol=1e-7)


def test_beta_zero_is_pure_decay():
    """With beta -> 0 (logit -40) only the decay acts:
    S_t = S0 diag(prod alpha) and o_t = s S0 diag(prod_{r<=t} alpha_r) q_t."""
    rng = _rng(3)
    L, d = 12, 128
    q, k, v, g, beta, A, dtb, S0 = _task(rng, L, d)
    beta[:] = -40.0
    o, S = ko.forward_task(q, k, v, g, beta, A, dtb, S0)
    gate = torch.exp(-5.0 * torch.sigmoid(math.exp(A) * (torch.from_numpy(g)
                                                         + torch.from_numpy(dtb)))).numpy()
    cp = np.cumprod(gate, axis=0)
    qn = torch.nn.functional.normalize(torch.from_numpy(q), dim=-1).numpy()
    for t in range(L):
        # rtol: normalize() places eps differently (~4e-9 relative)
        np.testing.assert_allclose(o[t], ko.SCALE * (S0 * cp[t][None, :]) @ qn[t],
                                   rtol=1e-7, atol=1e-14)
    np.testing.assert_allclose(S, S0 * cp[-1][None, :], rtol=0, atol=1e-14)


def test_basis_keys_replace_columns():
    """Textbook delta rule: with no decay (z = -40, so alpha = 1), beta = 1
    and key e_j, the update overwrites column j of the value-first state with
    v and leaves the other columns alone."""
    rng = _rng(4)
    d, L = 16, 10
    S = rng.standard_normal((d, d))
    S0 = S.copy()
    js = rng.integers(0, d, L)
    q = rng.standard_normal((L, d))
    k = np.zeros((L, d))
    k[np.arange(L), js] = 1000.0
    v = rng.standard_normal((L, d))
    g = np.full((L, d), -40.0)
    beta = np.full(L, 40.0)
    _, Sf = ko.forward_task(q, k, v, g, beta, 0.0, np.zeros(d), S0)
    for t in range(L):
        S[:, js[t]] = v[t]
    np.testing.assert_allclose(Sf, S, rtol=0, atol=1e-9)


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def test_linearity_in_state_and_values():
    """For fixed q, k, g, beta the map (S0, V) -> (O, S_T) is linear."""
    rng = _rng(5)
    q, k, v, g, beta, A, dtb, S0 = _task(rng, 15, 32)
    v2 = rng.standard_normal(v.shape)
    S2 = rng.standard_normal(S0.shape)
    a1, a2 = 0.7, -1.3
    o1, s1 = ko.forward_task(q, k, v, g, beta, A, dtb, S0)
    o2, s2 = ko.forward_task(q, k, v2, g, beta, A, dtb, S2)
    o3, s3 = ko.forward_task(q, k, a1 * v + a2 * v2, g, beta, A, dtb, a1 * S0 + a2 * S2)
    np.testing.assert_allclose(o3, a1 * o1 + a2 * o2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s3, a1 * s1 + a2 * s2, rtol=1e-12, atol=1e-12)


def test_state_continuity():
    """Running T tokens equals running T1 tokens and then T - T1 more from the
    state reached (the final state of one call is the initial state of the
    next)."""
    rng = _rng(6)
    q, k, v, g, beta, A, dtb, S0 = _task(rng, 29, 128)
    o, S = ko.forward_task(q, k, v, g, beta, A, dtb, S0)
    T1 = 13
    oa, Sa = ko.forward_task(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], A, dtb, S0)
    ob, Sb = ko.forward_task(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], A, dtb, Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sb, S, rtol=0, atol=1e-13)


def _problem_arrays(rng, lengths, packed, Hqk, Hv, d=128):
    B = 1 if packed else len(lengths)
    T = sum(lengths) if packed else lengths[0]
    N = len(lengths)
    return dict(
        q=rng.standard_normal((B, T, Hqk, d)), k=rng.standard_normal((B, T, Hqk, d)),
        v=rng.standard_normal((B, T, Hv, d)), g=rng.standard_normal((B, T, Hv, d)),
        beta=rng.standard_normal((B, T, Hv)), A_log=rng.uniform(0, 2, Hv),
        dt_bias=0.1 * rng.standard_normal((Hv, d)),
        initial_state=0.01 * rng.standard_normal((N, Hv, d, d)))


def test_packed_equals_fixed():
    """Packed layout (physical batch 1 plus cu_seqlens) and fixed layout
    (one sequence per batch row) describe the same computation
    ("flashinfer.kda_training", layout paragraph)."""
    rng = _rng(7)
    L, N, H = 9, 3, 2
    a = _problem_arrays(rng, [L] * N, False, H, H, d=16)
    o_f, s_f = oracle.forward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"],
                              a["dt_bias"], a["initial_state"], [L] * N, packed=False)
    pk = {n: a[n].reshape((1, N * L) + a[n].shape[2:]) for n in ("q", "k", "v", "g", "beta")}
    o_p, s_p = oracle.forward(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], a["A_log"],
                              a["dt_bias"], a["initial_state"], [L] * N, packed=True)
    np.testing.assert_array_equal(o_p.reshape(o_f.shape), o_f)
    np.testing.assert_array_equal(s_p, s_f)


def test_grouping_equals_repeated_heads():
    """Grouped heads (Hv a multiple of Hqk) equal the equal-head problem with q
    and k repeated per value head; grouped dq/dk are the sums over the value
    heads that share the q/k head (training-forward parameter v)."""
    rng = _rng(8)
    lengths = [7, 5]
    Hqk, G = 2, 3
    Hv = Hqk * G
    a = _problem_arrays(rng, lengths, True, Hqk, Hv, d=8)
    do = rng.standard_normal(a["v"].shape)
    dfs = 0.01 * rng.standard_normal(a["initial_state"].shape)
    rep = {n: np.repeat(a[n], G, axis=2) for n in ("q", "k")}
    args_g = (a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
              a["initial_state"])
    args_e = (rep["q"], rep["k"]) + args_g[2:]
    o_g, s_g = oracle.forward(*args_g, lengths, packed=True)
    o_e, s_e = oracle.forward(*args_e, lengths, packed=True)
    np.testing.assert_allclose(o_g, o_e, rtol=0, atol=1e-15)
    np.testing.assert_allclose(s_g, s_e, rtol=0, atol=1e-15)
    gg = oracle.backward(*args_g, do, dfs, lengths, packed=True)
    ge = oracle.backward(*args_e, do, dfs, lengths, packed=True)
    T = a["q"].shape[1]
    for i in (0, 1):  # dq, dk
        summed = ge[i].reshape(1, T, Hqk, G, 8).sum(axis=3)
        np.testing.assert_allclose(gg[i], summed, rtol=1e-12, atol=1e-15)
    for i in range(2, 8):
        np.testing.assert_allclose(gg[i], ge[i], rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------------------
# second formulation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("C", [1, 2, 4, 5, 16])
def test_chunked_equals_token_forward(C):
    """The chunked (WY / UT) form reaches the token recurrence's result; the
    last chunk is short (T = 11)."""
    rng = _rng(9)
    q, k, v, g, beta, A, dtb, S0 = _task(rng, 11, 128)
    o, S = ko.forward_task(q, k, v, g, beta, A, dtb, S0)
    oc, Sc = ko.chunk_forward_task(q, k, v, g, beta, A, dtb, S0, C=C)
    # fp64 round-off only (values are O(1))
    np.testing.assert_allclose(oc, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(Sc, S, rtol=0, atol=1e-13)


@pytest.mark.parametrize("C", [1, 3, 4, 16])
def test_chunk_adjoint_equals_token_adjoint(C):
    rng = _rng(10)
    L, d = 21, 128
    q, k, v, g, beta, A, dtb, S0 = _task(rng, L, d)
    do = rng.standard_normal((L, d))
    dSL = 0.01 * rng.standard_normal((d, d))
    gt = ko.backward_task(q, k, v, g, beta, A, dtb, S0, do, dSL)
    gc = ko.chunk_backward_task(q, k, v, g, beta, A, dtb, S0, do, dSL, C=C)
    for a, b in zip(gt, gc):
        a, b = np.asarray(a), np.asarray(b)
        np.testing.assert_allclose(b, a, rtol=1e-10, atol=1e-15)


# ---------------------------------------------------------------------------
# backward against finite differences
# ---------------------------------------------------------------------------
NAMES = ("q", "k", "v", "g", "beta", "A_log", "dt_bias", "S0")


def _loss(inp, do, dSL, fwd=ko.forward_task):
    o, S = fwd(*inp)
    return float((do * o).sum() + (dSL * S).sum())


def _fd_check(L, d, seed, bwd=ko.backward_task, fwd=ko.forward_task, h=1e-6, reps=2):
    rng = _rng(seed)
    inp = list(_task(rng, L, d))
    do = rng.standard_normal((L, d))
    dSL = rng.standard_normal((d, d))
    grads = bwd(*inp, do, dSL)
    worst = 0.0
    for i in range(8):
        for _ in range(reps):
            x = inp[i]
            u = rng.standard_normal(np.shape(x))
            plus = list(inp)
            minus = list(inp)
            if np.ndim(x) == 0:
                u = float(u)
                plus[i] = x + h * u
                minus[i] = x - h * u
            else:
                plus[i] = x + h * u
                minus[i] = x - h * u
            fd = (_loss(plus, do, dSL, fwd) - _loss(minus, do, dSL, fwd)) / (2 * h)
            an = float(np.sum(np.asarray(grads[i]) * u))
            rel = abs(fd - an) / max(abs(fd), abs(an), 1e-300)
            worst = max(worst, rel)
            if rel > 1e-6:
                return False, (NAMES[i], fd, an, rel)
    return True, worst


def test_backward_finite_differences_small():
    """All eight gradients of <do, o> + <dfinal_state, S_T> (the loss whose
    adjoints "recurrent_kda_backward" takes) against central differences at
    K=V=8, T=11."""
    ok, info = _fd_check(11, 8, 11)
    assert ok, info


def test_backward_finite_differences_full_width():
    """The same at the real head width K=V=128, T=4."""
    ok, info = _fd_check(4, 128, 12, reps=1)
    assert ok, info


def test_gradient_identities():
    """z = exp(A_log)(g + dt_bias) makes ddt_bias = sum_t dg and
    dA_log = sum dg * (g + dt_bias) exact identities."""
    rng = _rng(13)
    L, d = 17, 128
    inp = _task(rng, L, d)
    do = rng.standard_normal((L, d))
    dSL = rng.standard_normal((d, d))
    dq, dk, dv, dg, dbeta, dA, ddt, dS0 = ko.backward_task(*inp, do, dSL)
    q, k, v, g, beta, A, dtb, S0 = inp
    np.testing.assert_allclose(ddt, dg.sum(axis=0), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(dA, float((dg * (g + dtb[None, :])).sum()), rtol=1e-12)


def test_l2_scale_invariance():
    """The output depends on q and k only through their directions (up to
    eps), so dq . q and dk . k vanish per token."""
    rng = _rng(14)
    L, d = 9, 128
    inp = _task(rng, L, d)
    do = rng.standard_normal((L, d))
    dSL = rng.standard_normal((d, d))
    dq, dk = ko.backward_task(*inp, do, dSL)[:2]
    q, k = inp[0], inp[1]
    rq = np.abs((dq * q).sum(axis=1)) / (np.linalg.norm(dq, axis=1) * np.linalg.norm(q, axis=1))
    rk = np.abs((dk * k).sum(axis=1)) / (np.linalg.norm(dk, axis=1) * np.linalg.norm(k, axis=1))
    assert rq.max() < 1e-7 and rk.max() < 1e-7


def test_whole_problem_driver_matches_tasks():
    """The packed driver slices sequences by cu_seqlens and heads by the
    grouping rule; spot-check one task against a direct call."""
    rng = _rng(15)
    lengths = [5, 11, 3]
    a = _problem_arrays(rng, lengths, True, 2, 4, d=16)
    o, s = oracle.forward(a["q"], a["k"], a["v"], a["g"], a["beta"], a["A_log"], a["dt_bias"],
                          a["initial_state"], lengths, packed=True)
    n, h = 1, 3
    t0 = 5
    sl = slice(t0, t0 + 11)
    ot, st = ko.forward_task(a["q"][0, sl, 1], a["k"][0, sl, 1], a["v"][0, sl, h],
                             a["g"][0, sl, h], a["beta"][0, sl, h], float(a["A_log"][h]),
                             a["dt_bias"][h], a["initial_state"][n, h])
    np.testing.assert_array_equal(o[0, sl, h], ot)
    np.testing.assert_array_equal(s[n, h], st)
