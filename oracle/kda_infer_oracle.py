"""FP64 CPU oracle of the recurrent KDA inference forward with its gate, beta
and norm options and an in-place state pool.

TEST INFRASTRUCTURE ONLY, like kda_oracle: only the tests, the smoke check
and the benchmark's CPU-baseline leg may use it. It shares no code with the
HIP kernels.

Source: page "flashinfer.kda.recurrent_kda", parameters:
  * use_qk_l2norm_in_kernel: q and k are L2-normalised (epsilon 1e-6, as in
    the training pages) when set, used as given otherwise;
  * use_gate_in_kernel: when set, the per-K-channel log-decay is
    lower_bound * sigmoid(exp(A_log) * (g + dt_bias)) (the lower_bound form;
    the softplus form's formula is not on the pages and is not modelled);
    when clear, g is already the log-space decay, so the decay is exp(g);
  * beta_is_logit: beta passes through a sigmoid when set and is used as
    given otherwise;
  * initial_state with ssm_state_indices: a value-first state pool
    [P, Hv, V, K] whose slot indices[n] holds sequence n's initial state and
    receives its final state in place; slots no sequence names are left as
    they were;
  * state_checkpoints with checkpoint_every_n_tokens E: per sequence,
    ceil(L / E) states, row j being the state before token j*E (row 0 the
    initial state), stored from the sequence's cumulative start on;
  * num_spec_tokens S with ssm_state_indices [N, 1+S] and num_accepted_tokens:
    every sequence has 1+S tokens; its initial state is slot [n, a-1], a the
    accepted count of the previous round clamped to [1, 1+S] (slot [n, 0]
    without counts), and the state after token s goes to slot [n, s]
    (reading: the per-token slots are the checkpoints a later round resumes
    from);
  * initial_state_source with initial_state_indices: a read-only pool whose
    slot source_indices[n] replaces the state sequence n starts from.
The recurrence itself is kda_oracle.recurrence (decay, delta-rule update from
the decayed state, read-out from the updated state).

Readings (listed in the design notes): dt_bias may be absent and then counts
as zero; the pool is returned in FP64 (the kernel stores BF16, and the tests
compare at the BF16 bar).
"""
from __future__ import annotations

import math

import numpy as np

from oracle.kda_oracle import EPS, SCALE, _np64, _sigmoid, _slices, recurrence


def infer_prologue(q, k, g, beta, A_log_h, dt_bias_h, use_qk_l2norm=True,
                   use_gate_in_kernel=False, lower_bound=None, beta_is_logit=False, eps=EPS):
    """Per-token prologue of one (sequence, value head) with the inference
    options. q, k, g: [L, d]; beta: [L]; A_log_h: scalar or None; dt_bias_h:
    [d] or None. Returns (qn, kn, alpha, b)."""
    if use_qk_l2norm:
        qn = q / np.sqrt((q * q).sum(axis=-1, keepdims=True) + eps)
        kn = k / np.sqrt((k * k).sum(axis=-1, keepdims=True) + eps)
    else:
        qn, kn = q, k
    if use_gate_in_kernel:
        if lower_bound is None:
            raise ValueError("the softplus gate form is not modelled: pass lower_bound")
        bias = 0.0 if dt_bias_h is None else dt_bias_h[None, :]
        lam = lower_bound * _sigmoid(math.exp(A_log_h) * (g + bias))
    else:
        lam = g
    alpha = np.exp(lam)
    b = _sigmoid(beta) if beta_is_logit else beta
    return qn, kn, alpha, b


def infer_forward(q, k, v, g, beta, A_log, dt_bias, pool, lengths, packed, indices=None,
                  scale=None, use_qk_l2norm=True, use_gate_in_kernel=False, lower_bound=None,
                  beta_is_logit=False, checkpoint_every=0, num_spec_tokens=0,
                  num_accepted=None, source=None, source_indices=None):
    """Whole-problem inference forward. q, k [B,T,Hqk,d]; v, g [B,T,Hv,d];
    beta [B,T,Hv]; A_log [Hv] or None; dt_bias [Hv,d] or None; pool
    [P,Hv,d,d]; indices [N] or None (slot n).

    Returns (o [B,T,Hv,d], new_pool [P,Hv,d,d]) in FP64, and with
    checkpoint_every = E > 0 also the checkpoints [sum ceil(L/E), Hv, d, d]."""
    scale = SCALE if scale is None else float(scale)
    Hqk, Hv = q.shape[2], v.shape[2]
    G = Hv // Hqk
    N = len(lengths)
    S = int(num_spec_tokens)
    if S:
        slots = [[int(x) for x in row] for row in indices]
        if any(int(L) != 1 + S for L in lengths):
            raise ValueError("speculative decode needs 1+S tokens per sequence")
        flat = [x for row in slots for x in row]
        acc = [1] * N if num_accepted is None else [min(max(int(a), 1), 1 + S) for a in num_accepted]
        idx = [slots[n][acc[n] - 1] for n in range(N)]
    else:
        idx = list(range(N)) if indices is None else [int(i) for i in indices]
        flat = idx
    if len(set(flat)) != len(flat):
        raise ValueError("pool slots must be distinct")
    o = np.full(tuple(v.shape), np.nan)
    new_pool = _np64(pool).copy()
    E = int(checkpoint_every)
    starts = np.concatenate([[0], np.cumsum([-(-int(L) // E) for L in lengths])]) if E else None
    ckpts = np.full((int(starts[-1]), Hv) + tuple(pool.shape[2:]), np.nan) if E else None
    for (n, b, t0, L) in _slices(lengths, packed):
        s = slice(t0, t0 + L)
        for h in range(Hv):
            hq = h // G
            qn, kn, alpha, bb = infer_prologue(
                _np64(q[b, s, hq]), _np64(k[b, s, hq]), _np64(g[b, s, h]), _np64(beta[b, s, h]),
                None if A_log is None else float(A_log[h]),
                None if dt_bias is None else _np64(dt_bias[h]),
                use_qk_l2norm, use_gate_in_kernel, lower_bound, beta_is_logit)
            S0 = _np64(pool[idx[n], h]) if source is None else _np64(source[int(source_indices[n]), h])
            on, Sn, states = recurrence(qn, kn, _np64(v[b, s, h]), alpha, bb, S0, scale,
                                        keep_states=True)
            o[b, s, h] = on
            if S:
                for t in range(1 + S):
                    new_pool[slots[n][t], h] = states[t + 1]   # after token t
            else:
                new_pool[idx[n], h] = Sn
            if E:
                for j in range(-(-L // E)):
                    ckpts[starts[n] + j, h] = states[j * E]   # before token j*E
    if E:
        return o, new_pool, ckpts
    return o, new_pool
