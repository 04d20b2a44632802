"""FP64 CPU oracle of the recurrent KDA training recurrence.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP kernels.

Sources (FlashInfer documentation pages):
  * "flashinfer.kda_backward.recurrent_kda_backward", description: q and k
    are L2-normalised with epsilon 1e-6; the per-channel decay is
    exp(lower_bound * sigmoid(exp(A_log) * (g + dt_bias))); beta passes
    through a sigmoid; the loss adjoints are `do` for the token output and
    `dfinal_state` for the final state; the gradients come back in the
    order (dq, dk, dv, dg, dbeta, dA_log, ddt_bias, dinitial_state).
  * "flashinfer.kda_training.recurrent_kda_training_forward", parameters:
    value-first FP32 state [N, Hv, V, K], grouped heads (Hv a multiple of
    Hqk), packed layout through cu_seqlens, scale fixed at 1/sqrt(128),
    lower bound fixed at -5.
  * "flashinfer.kda_training", paragraphs 3-4: every sequence is
    non-empty; packed and fixed layouts; no alignment requirement.

The pages never print the recurrence itself. The reading used here (decay
first, then the delta-rule update computed from the decayed state, then the
read-out from the updated state) is the plainest one that the pages'
per-K-dimension gate, value-first state and delta-rule learning rate admit:

    P_t = S_{t-1} diag(alpha_t)
    e_t = v_t - P_t k_t
    S_t = P_t + beta_t e_t k_t^T
    o_t = scale * S_t q_t

Other readings, each immaterial or fixed by self-consistency only:
  * L2 norm: x / sqrt(|x|^2 + eps).
  * Head grouping: value head h reads q/k head h // (Hv / Hqk).
  * A_log and dt_bias are indexed by value head.
  * dq, dk, dg, dbeta are gradients with respect to the raw inputs
    (pre-normalisation q/k, raw gate, beta logits).

Functions
  prologue          per-token normalisation, gate and beta
  forward_task      token-by-token forward of one (sequence, value head)
  backward_task     exact vector-Jacobian product of forward_task, by the
                    hand-derived token adjoint (reverse-mode of the four
                    update equations above), with FP64 state checkpoints
  chunk_forward_task / chunk_backward_task
                    the same maps in chunked (WY / UT) form; a second
                    formulation used only to cross-check the first and to
                    give stage-level references
  forward / backward
                    whole-problem drivers over all tasks, optionally on a
                    process pool

Parity pins (tests/test_oracle_pins.py): closed forms for a single token, for
beta -> 0 and for the basis-key delta rule; the S k = v invariant at beta = 1;
linearity; state continuity; packed == fixed; grouping; chunk == token; the
backward against central finite differences and exact gradient identities.
The q/k head mapping and the epsilon placement are "parity unpinned": they
are self-consistent only.
"""
from __future__ import annotations

import math
import os
from typing import Optional

import numpy as np

EPS = 1e-6
LOWER_BOUND = -5.0
SCALE = 1.0 / math.sqrt(128.0)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


# ---------------------------------------------------------------------------
# prologue
# ---------------------------------------------------------------------------
def prologue(q, k, g, beta, A_log_h, dt_bias_h, lb=LOWER_BOUND, eps=EPS):
    """Per-token prologue ("recurrent_kda_backward" description).

    q, k, g: [L, d]; beta: [L] raw logits; A_log_h: scalar; dt_bias_h: [d].
    Returns (qn, kn, lam, alpha, b, z) with lam = lb*sigmoid(z) the log-decay,
    alpha = exp(lam), b = sigmoid(beta).
    """
    qn = q / np.sqrt((q * q).sum(axis=-1, keepdims=True) + eps)
    kn = k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + eps)
    z = math.exp(A_log_h) * (g + dt_bias_h[None, :])
    lam = lb * _sigmoid(z)
    alpha = np.exp(lam)
    b = _sigmoid(beta)
    return qn, kn, lam, alpha, b, z


# ---------------------------------------------------------------------------
# token-by-token forward
# ---------------------------------------------------------------------------
def recurrence(qn, kn, v, alpha, b, S0, scale=SCALE, keep_states=False):
    """The recurrence on prologue outputs. Returns (o [L, dv], S_L[, states])."""
    S = S0.copy()
    L = qn.shape[0]
    o = np.empty((L, v.shape[1]))
    states = [S.copy()] if keep_states else None
    for t in range(L):
        P = S * alpha[t][None, :]
        e = v[t] - P @ kn[t]
        S = P + b[t] * np.outer(e, kn[t])
        o[t] = scale * (S @ qn[t])
        if keep_states:
            states.append(S.copy())
    if keep_states:
        return o, S, states
    return o, S


def forward_task(q, k, v, g, beta, A_log_h, dt_bias_h, S0, scale=SCALE,
                 lb=LOWER_BOUND, eps=EPS):
    """One (sequence, value head): o [L, d] (FP64, unrounded) and S_L [d, d]."""
    qn, kn, lam, alpha, b, z = prologue(q, k, g, beta, A_log_h, dt_bias_h, lb, eps)
    return recurrence(qn, kn, v, alpha, b, S0, scale)


# ---------------------------------------------------------------------------
# token adjoint
# ---------------------------------------------------------------------------
def _l2_backward(x, dxn, eps=EPS):
    """Gradient through xn = x / sqrt(|x|^2 + eps), row-wise."""
    r = 1.0 / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)
    xn = x * r
    return r * (dxn - xn * (xn * dxn).sum(axis=-1, keepdims=True))


def recurrence_backward(qn, kn, v, alpha, b, S0, do, dSL, scale=SCALE, seg=64):
    """Reverse-mode through `recurrence`.

    Returns (dqn, dkn, dv, dalpha, db, dS0). The forward states are kept at
    every `seg` tokens and each segment is recomputed before it is walked
    backwards, so memory stays at `seg` states.
    """
    L = qn.shape[0]
    ck = []
    S = S0.copy()
    for t in range(L):
        if t % seg == 0:
            ck.append(S.copy())
        P = S * alpha[t][None, :]
        e = v[t] - P @ kn[t]
        S = P + b[t] * np.outer(e, kn[t])
    dqn = np.zeros_like(qn)
    dkn = np.zeros_like(kn)
    dv = np.zeros_like(v)
    dalpha = np.zeros_like(alpha)
    db = np.zeros_like(b)
    Sh = dSL.copy()  # adjoint of the current state
    for si in range(len(ck) - 1, -1, -1):
        t0 = si * seg
        t1 = min(L, t0 + seg)
        states = [ck[si]]
        S = ck[si]
        for t in range(t0, t1):
            P = S * alpha[t][None, :]
            e = v[t] - P @ kn[t]
            S = P + b[t] * np.outer(e, kn[t])
            states.append(S)
        for t in range(t1 - 1, t0 - 1, -1):
            S_prev = states[t - t0]
            S_t = states[t - t0 + 1]
            P = S_prev * alpha[t][None, :]
            e = v[t] - P @ kn[t]
            # o_t = scale * S_t q_t
            dqn[t] = scale * (S_t.T @ do[t])
            Sh = Sh + scale * np.outer(do[t], qn[t])
            # S_t = P + b e k^T, e = v - P k
            Sk = Sh @ kn[t]
            dv[t] = b[t] * Sk
            db[t] = e @ Sk
            dkn[t] = b[t] * (Sh.T @ e - P.T @ Sk)
            dP = Sh - b[t] * np.outer(Sk, kn[t])
            # P = S_prev diag(alpha)
            dalpha[t] = (dP * S_prev).sum(axis=0)
            Sh = dP * alpha[t][None, :]
    return dqn, dkn, dv, dalpha, db, Sh


def prologue_backward(q, k, g, beta, A_log_h, dt_bias_h, dqn, dkn, dlam, db,
                      lb=LOWER_BOUND, eps=EPS):
    """Chain rule through `prologue`, given the adjoint of the log-decay lam.

    Returns (dq, dk, dg, dbeta, dA_log_h, ddt_bias_h)."""
    eA = math.exp(A_log_h)
    z = eA * (g + dt_bias_h[None, :])
    sz = _sigmoid(z)
    dz = lb * dlam * sz * (1.0 - sz)
    dg = eA * dz
    ddt = dg.sum(axis=0)
    dA = float((dz * z).sum())
    bb = _sigmoid(beta)
    dbeta = db * bb * (1.0 - bb)
    dq = _l2_backward(q, dqn, eps)
    dk = _l2_backward(k, dkn, eps)
    return dq, dk, dg, dbeta, dA, ddt


def backward_task(q, k, v, g, beta, A_log_h, dt_bias_h, S0, do, dSL,
                  scale=SCALE, lb=LOWER_BOUND, eps=EPS):
    """Vector-Jacobian product of forward_task for the loss
    <do, o> + <dSL, S_L>. Returns (dq, dk, dv, dg, dbeta, dA_log_h,
    ddt_bias_h, dS0); dq and dk are this value head's contribution to its
    q/k head."""
    qn, kn, lam, alpha, b, z = prologue(q, k, g, beta, A_log_h, dt_bias_h, lb, eps)
    dqn, dkn, dv, dalpha, db, dS0 = recurrence_backward(qn, kn, v, alpha, b, S0, do, dSL, scale)
    dlam = dalpha * alpha
    dq, dk, dg, dbeta, dA, ddt = prologue_backward(q, k, g, beta, A_log_h, dt_bias_h,
                                                   dqn, dkn, dlam, db, lb, eps)
    return dq, dk, dv, dg, dbeta, dA, ddt, dS0


# ---------------------------------------------------------------------------
# chunked form (second formulation, cross-check only)
# ---------------------------------------------------------------------------
def chunk_quantities(qn, kn, v, lam, b, scale=SCALE):
    """Intra-chunk quantities of one chunk (rows = tokens of the chunk).

    With gc = cumsum(lam) and Gamma = exp(gc):
      Qg = qn*Gamma, Kg = kn*Gamma, Ki = kn/Gamma, Kt = kn*exp(gc[-1]-gc),
      Akk = strictly-lower(Kg Ki^T), Aqk = lower(Qg Ki^T),
      T = (I + diag(b) Akk)^-1, W = T diag(b) Kg, Ut = T diag(b) v.
    """
    gc = np.cumsum(lam, axis=0)
    Gam = np.exp(gc)
    gC = gc[-1]
    Qg = qn * Gam
    Kg = kn * Gam
    Ki = kn * np.exp(-gc)
    Kt = kn * np.exp(gC[None, :] - gc)
    n = qn.shape[0]
    Akk = np.tril(Kg @ Ki.T, -1)
    Aqk = np.tril(Qg @ Ki.T, 0)
    T = np.linalg.inv(np.eye(n) + b[:, None] * Akk)
    W = T @ (b[:, None] * Kg)
    Ut = T @ (b[:, None] * v)
    return dict(gc=gc, gC=gC, Qg=Qg, Kg=Kg, Ki=Ki, Kt=Kt, Akk=Akk, Aqk=Aqk,
                T=T, W=W, Ut=Ut)


def chunk_recurrence(qn, kn, v, lam, b, S0, C, scale=SCALE, keep_states=False):
    """Chunked evaluation of `recurrence`; the last chunk may be short.

    Per chunk with start state S0:
      U = Ut - W S0^T,  O = scale (Qg S0^T + Aqk U),
      S_C = S0 diag(exp(gc[-1])) + U^T Kt.
    """
    L = qn.shape[0]
    S = S0.copy()
    o = np.empty((L, v.shape[1]))
    states = [S.copy()] if keep_states else None
    for c0 in range(0, L, C):
        sl = slice(c0, min(L, c0 + C))
        cq = chunk_quantities(qn[sl], kn[sl], v[sl], lam[sl], b[sl], scale)
        U = cq["Ut"] - cq["W"] @ S.T
        o[sl] = scale * (cq["Qg"] @ S.T + cq["Aqk"] @ U)
        S = S * np.exp(cq["gC"])[None, :] + U.T @ cq["Kt"]
        if keep_states:
            states.append(S.copy())
    if keep_states:
        return o, S, states
    return o, S


def chunk_forward_task(q, k, v, g, beta, A_log_h, dt_bias_h, S0, C=16, scale=SCALE,
                       lb=LOWER_BOUND, eps=EPS):
    qn, kn, lam, alpha, b, z = prologue(q, k, g, beta, A_log_h, dt_bias_h, lb, eps)
    return chunk_recurrence(qn, kn, v, lam, b, S0, C, scale)


def chunk_recurrence_backward(qn, kn, v, lam, b, S0, do, dSL, C, scale=SCALE):
    """Reverse-mode through `chunk_recurrence`, chunk by chunk.

    Returns (dqn, dkn, dv, dlam, db, dS0)."""
    L = qn.shape[0]
    _, _, states = chunk_recurrence(qn, kn, v, lam, b, S0, C, scale, keep_states=True)
    dqn = np.zeros_like(qn)
    dkn = np.zeros_like(kn)
    dv = np.zeros_like(v)
    dlam = np.zeros_like(lam)
    db = np.zeros_like(b)
    dS = dSL.copy()
    starts = list(range(0, L, C))
    for ci in range(len(starts) - 1, -1, -1):
        c0 = starts[ci]
        sl = slice(c0, min(L, c0 + C))
        S0c = states[ci]
        cq = chunk_quantities(qn[sl], kn[sl], v[sl], lam[sl], b[sl], scale)
        Qg, Kg, Ki, Kt = cq["Qg"], cq["Kg"], cq["Ki"], cq["Kt"]
        Akk, Aqk, T, W = cq["Akk"], cq["Aqk"], cq["T"], cq["W"]
        gc, gC = cq["gc"], cq["gC"]
        bc = b[sl]
        vc = v[sl]
        dO = do[sl]
        U = cq["Ut"] - W @ S0c.T
        eC = np.exp(gC)
        # S_C = S0 diag(eC) + U^T Kt
        dS0 = dS * eC[None, :]
        dgC = (dS * S0c).sum(axis=0) * eC
        dU = Kt @ dS.T
        dKt = U @ dS
        # O = scale (Qg S0^T + Aqk U)
        dQg = scale * (dO @ S0c)
        dS0 = dS0 + scale * (dO.T @ Qg)
        dAqk = np.tril(scale * (dO @ U.T), 0)
        dU = dU + scale * (Aqk.T @ dO)
        # U = Ut - W S0^T
        dUt = dU
        dW = -(dU @ S0c)
        dS0 = dS0 - dU.T @ W
        # Ut = T diag(b) v ; W = T diag(b) Kg
        Bv = bc[:, None] * vc
        Bk = bc[:, None] * Kg
        dT = dUt @ Bv.T + dW @ Bk.T
        dBv = T.T @ dUt
        dBk = T.T @ dW
        dvc = bc[:, None] * dBv
        dbc = (dBv * vc).sum(axis=1) + (dBk * Kg).sum(axis=1)
        dKg = bc[:, None] * dBk
        # T = (I + diag(b) Akk)^-1
        dM = -T.T @ dT @ T.T
        dAkk = np.tril(bc[:, None] * dM, -1)
        dbc = dbc + (dM * Akk).sum(axis=1)
        # Akk = strict-lower(Kg Ki^T), Aqk = lower(Qg Ki^T)
        dKg = dKg + dAkk @ Ki
        dKi = dAkk.T @ Kg + dAqk.T @ Qg
        dQg = dQg + dAqk @ Ki
        # exponential factors
        Gam = np.exp(gc)
        dkc = dKt * np.exp(gC[None, :] - gc) + dKg * Gam + dKi * np.exp(-gc)
        dqc = dQg * Gam
        dg = -dKt * Kt + dKg * Kg - dKi * Ki + dQg * Qg
        dgC = dgC + (dKt * Kt).sum(axis=0)
        dg[-1] += dgC
        dlam[sl] = np.cumsum(dg[::-1], axis=0)[::-1]
        dqn[sl] = dqc
        dkn[sl] = dkc
        dv[sl] = dvc
        db[sl] = dbc
        dS = dS0
    return dqn, dkn, dv, dlam, db, dS


def chunk_backward_task(q, k, v, g, beta, A_log_h, dt_bias_h, S0, do, dSL, C=16,
                        scale=SCALE, lb=LOWER_BOUND, eps=EPS):
    qn, kn, lam, alpha, b, z = prologue(q, k, g, beta, A_log_h, dt_bias_h, lb, eps)
    dqn, dkn, dv, dlam, db, dS0 = chunk_recurrence_backward(qn, kn, v, lam, b, S0, do, dSL,
                                                            C, scale)
    dq, dk, dg, dbeta, dA, ddt = prologue_backward(q, k, g, beta, A_log_h, dt_bias_h,
                                                   dqn, dkn, dlam, db, lb, eps)
    return dq, dk, dv, dg, dbeta, dA, ddt, dS0


# ---------------------------------------------------------------------------
# whole-problem drivers
# ---------------------------------------------------------------------------
def _np64(t):
    if t is None:
        return None
    try:
        import torch
        if isinstance(t, torch.Tensor):
            return t.detach().to("cpu", dtype=torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(t, dtype=np.float64)


def _slices(lengths, packed):
    out = []
    t0 = 0
    for n, L in enumerate(lengths):
        if packed:
            out.append((n, 0, t0, int(L)))
            t0 += int(L)
        else:
            out.append((n, n, 0, int(L)))
    return out


def task_list(lengths, packed, Hqk, Hv, tasks=None):
    """All (n, h) tasks, or the given subset, with their token slices."""
    sl = _slices(lengths, packed)
    if tasks is None:
        tasks = [(n, h) for n in range(len(lengths)) for h in range(Hv)]
    G = Hv // Hqk
    return [(n, h, h // G) + sl[n][1:] for (n, h) in tasks]


def _fwd_job(args):
    n, h, q, k, v, g, beta, A, dtb, S0 = args
    o, S = forward_task(q, k, v, g, beta, A, dtb, S0)
    return n, h, o, S


def _bwd_job(args):
    n, h, q, k, v, g, beta, A, dtb, S0, do, dSL = args
    return (n, h) + tuple(backward_task(q, k, v, g, beta, A, dtb, S0, do, dSL))


def _worker_init():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass


def _map(fn, jobs, workers):
    if workers is None or workers <= 1 or len(jobs) <= 1:
        return [fn(j) for j in jobs]
    import multiprocessing as mp
    ctx = mp.get_context("fork")
    with ctx.Pool(workers, initializer=_worker_init) as pool:
        return pool.map(fn, jobs, chunksize=1)


def _task_jobs(tl, q, k, v, g, beta, A_log, dt_bias, initial_state, do=None, dfinal_state=None):
    # each job carries FP64 copies of its own slices only
    jobs = []
    for (n, h, hq, b, t0, L) in tl:
        s = slice(t0, t0 + L)
        job = (n, h, _np64(q[b, s, hq]), _np64(k[b, s, hq]), _np64(v[b, s, h]), _np64(g[b, s, h]),
               _np64(beta[b, s, h]), float(A_log[h]), _np64(dt_bias[h]), _np64(initial_state[n, h]))
        if do is not None:
            job = job + (_np64(do[b, s, h]), _np64(dfinal_state[n, h]))
        jobs.append(job)
    return jobs


def forward_tasks(q, k, v, g, beta, A_log, dt_bias, initial_state, lengths, packed, tasks,
                  workers=None):
    """Forward of the given (n, h) tasks: {(n, h): (o [L, d], S_L [d, d])} in FP64.
    Arrays follow the training API's tensor contract (see `forward`)."""
    Hqk, Hv = q.shape[2], v.shape[2]
    tl = task_list(lengths, packed, Hqk, Hv, tasks)
    jobs = _task_jobs(tl, q, k, v, g, beta, A_log, dt_bias, initial_state)
    return {(n, h): (o, S) for n, h, o, S in _map(_fwd_job, jobs, workers)}


def backward_tasks(q, k, v, g, beta, A_log, dt_bias, initial_state, do, dfinal_state,
                   lengths, packed, tasks, workers=None):
    """Backward of the given (n, h) tasks: {(n, h): (dq, dk, dv, dg, dbeta,
    dA_log_h, ddt_bias_h, dS0)} in FP64, where dq and dk are this value head's
    contribution to its q/k head and dA_log_h, ddt_bias_h this task's share."""
    Hqk, Hv = q.shape[2], v.shape[2]
    tl = task_list(lengths, packed, Hqk, Hv, tasks)
    jobs = _task_jobs(tl, q, k, v, g, beta, A_log, dt_bias, initial_state, do, dfinal_state)
    return {(r[0], r[1]): r[2:] for r in _map(_bwd_job, jobs, workers)}


def forward(q, k, v, g, beta, A_log, dt_bias, initial_state, lengths, packed,
            tasks=None, workers=None):
    """Whole-problem forward. Arrays follow the training API's tensor contract
    (q, k [B,T,Hqk,d]; v, g [B,T,Hv,d]; beta [B,T,Hv]; A_log [Hv];
    dt_bias [Hv,d]; initial_state [N,Hv,d,d]).

    Returns (o [B,T,Hv,d], final_state [N,Hv,d,d]) in FP64. With `tasks`
    (a list of (n, h)) only those tasks are computed and the rest of the
    outputs is NaN."""
    Hqk, Hv = q.shape[2], v.shape[2]
    tl = task_list(lengths, packed, Hqk, Hv, tasks)
    res = forward_tasks(q, k, v, g, beta, A_log, dt_bias, initial_state, lengths, packed,
                        [(n, h) for (n, h, *_r) in tl], workers)
    o = np.full(tuple(v.shape), np.nan)
    fs = np.full(tuple(initial_state.shape), np.nan)
    for (n, h, hq, b, t0, L) in tl:
        on, Sn = res[(n, h)]
        o[b, t0:t0 + L, h] = on
        fs[n, h] = Sn
    return o, fs


def backward(q, k, v, g, beta, A_log, dt_bias, initial_state, do, dfinal_state,
             lengths, packed, tasks=None, workers=None):
    """Whole-problem backward: (dq, dk, dv, dg, dbeta, dA_log, ddt_bias,
    dinitial_state) in FP64. dq/dk sum the contributions of the value heads
    that share a q/k head; dA_log and ddt_bias sum over every sequence and
    token. With `tasks`, only those tasks contribute (outputs of other tasks
    are NaN; dq/dk/dA_log/ddt_bias hold partial sums)."""
    Hqk, Hv = q.shape[2], v.shape[2]
    tl = task_list(lengths, packed, Hqk, Hv, tasks)
    res = backward_tasks(q, k, v, g, beta, A_log, dt_bias, initial_state, do, dfinal_state,
                         lengths, packed, [(n, h) for (n, h, *_r) in tl], workers)
    fill = np.nan if tasks is not None else 0.0
    dq = np.zeros(tuple(q.shape))
    dk = np.zeros(tuple(k.shape))
    dv = np.full(tuple(v.shape), fill)
    dg = np.full(tuple(g.shape), fill)
    dbeta = np.full(tuple(beta.shape), fill)
    dA = np.zeros(tuple(A_log.shape))
    ddt = np.zeros(tuple(dt_bias.shape))
    dS0 = np.full(tuple(initial_state.shape), fill)
    for (n, h, hq, b, t0, L) in tl:
        dqt, dkt, dvt, dgt, dbt, dAt, ddtt, dS0t = res[(n, h)]
        s = slice(t0, t0 + L)
        dq[b, s, hq] += dqt
        dk[b, s, hq] += dkt
        dv[b, s, h] = dvt
        dg[b, s, h] = dgt
        dbeta[b, s, h] = dbt
        dA[h] += dAt
        ddt[h] += ddtt
        dS0[n, h] = dS0t
    return dq, dk, dv, dg, dbeta, dA, ddt, dS0


def default_workers(cap=16):
    """Worker processes for the task pool: the CPUs this process may use, at
    most `cap`."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, cap))
