"""Pins of the FP64 inference oracle (oracle/kda_infer_oracle.py) to facts the
pages and the mathematics fix, independent of the oracle's own code paths
(page "flashinfer.kda.recurrent_kda", parameters use_qk_l2norm_in_kernel,
use_gate_in_kernel, lower_bound, beta_is_logit, initial_state and
ssm_state_indices).

* With every option at the training pages' setting (norm on, in-kernel gate
  with lower bound -5, beta as a logit) and the pool in sequence order, the
  result is the training oracle's, which its own pins tie to the pages.
* Log-space gate with beta = 0: no update, so the state is the initial state
  times exp(sum of g) per key channel, and each output is the closed form
  scale * S0 diag(exp(cumsum g)) q.
* Beta used as given, beta = 1, no decay (g = 0), unit keys: the delta rule
  stores v exactly along k, so with q = k every output is scale * v.
* Norm off: a key of length 2 doubles the stored value (closed form of one
  token from a zero state), and unit inputs give the norm-on result up to
  the epsilon (relative 5e-7).
* Pool: slots named by the indices receive the final states, in place; all
  other slots are returned unchanged.
* Checkpoints: row 0 of a sequence is its initial state, and row j equals
  the final state of the same sequence cut after j*E tokens.
* Speculative decode: slot [n, s] receives the state after token s, equal to
  a plain run over the first s+1 tokens from the accepted slot's state.
* Source pool: starting from source slot j equals starting from a pool whose
  slot holds the same state; the source itself is not written.
"""
import math

import numpy as np
import pytest

from oracle import kda_infer_oracle as kio
from oracle import kda_oracle as ko

D = 128
SCALE = 1.0 / math.sqrt(D)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def test_training_settings_reproduce_training_oracle():
    rng = np.random.default_rng(11)
    lengths, Hqk, Hv = [5, 9], 1, 2
    T = sum(lengths)
    q, k = _rand(rng, 1, T, Hqk, D), _rand(rng, 1, T, Hqk, D)
    v, g = _rand(rng, 1, T, Hv, D), _rand(rng, 1, T, Hv, D)
    beta = _rand(rng, 1, T, Hv)
    A_log, dt_bias = 2 * rng.random(Hv), 0.1 * _rand(rng, Hv, D)
    S0 = 0.01 * _rand(rng, 2, Hv, D, D)
    o_t, fs_t = ko.forward(q, k, v, g, beta, A_log, dt_bias, S0, lengths, packed=True)
    o_i, pool = kio.infer_forward(q, k, v, g, beta, A_log, dt_bias, S0, lengths, packed=True,
                                  use_qk_l2norm=True, use_gate_in_kernel=True, lower_bound=-5.0,
                                  beta_is_logit=True)
    assert np.array_equal(o_i, o_t) and np.array_equal(pool, fs_t)


def test_log_space_gate_closed_form_without_update():
    rng = np.random.default_rng(12)
    L = 7
    q, k, v = _rand(rng, 1, L, 1, D), _rand(rng, 1, L, 1, D), _rand(rng, 1, L, 1, D)
    g = -2.0 * rng.random((1, L, 1, D))        # log-space decays in (-2, 0]
    beta = np.zeros((1, L, 1))                 # used as given: no update
    S0 = _rand(rng, 1, 1, D, D)
    o, pool = kio.infer_forward(q, k, v, g, beta, None, None, S0, [L], packed=True,
                                use_gate_in_kernel=False, beta_is_logit=False)
    cum = np.cumsum(g[0, :, 0], axis=0)        # [L, D]
    for t in range(L):
        St = S0[0, 0] * np.exp(cum[t])[None, :]
        qn = q[0, t, 0] / math.sqrt(q[0, t, 0] @ q[0, t, 0] + 1e-6)
        np.testing.assert_allclose(o[0, t, 0], SCALE * St @ qn, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(pool[0, 0], S0[0, 0] * np.exp(cum[-1])[None, :], rtol=1e-12)


def test_beta_as_given_stores_value_along_unit_key():
    rng = np.random.default_rng(13)
    L = 6
    k = _unit(_rand(rng, 1, L, 1, D))
    v = _rand(rng, 1, L, 1, D)
    g = np.zeros((1, L, 1, D))                 # log-space 0: no decay
    beta = np.ones((1, L, 1))                  # used as given
    S0 = _rand(rng, 1, 1, D, D)
    o, _ = kio.infer_forward(k, k, v, g, beta, None, None, S0, [L], packed=True,
                             use_qk_l2norm=False, use_gate_in_kernel=False, beta_is_logit=False)
    np.testing.assert_allclose(o[0, :, 0], SCALE * v[0, :, 0], rtol=1e-10, atol=1e-12)


def test_norm_off_uses_keys_as_given():
    rng = np.random.default_rng(14)
    u = _unit(_rand(rng, 1, 1, 1, D))
    v = _rand(rng, 1, 1, 1, D)
    g = np.zeros((1, 1, 1, D))
    beta = np.ones((1, 1, 1))
    S0 = np.zeros((1, 1, D, D))
    # one token from a zero state: S = beta v k^T, o = scale S q = scale v (k.q)
    o, _ = kio.infer_forward(u, 2 * u, v, g, beta, None, None, S0, [1], packed=True,
                             use_qk_l2norm=False, use_gate_in_kernel=False, beta_is_logit=False)
    np.testing.assert_allclose(o[0, 0, 0], SCALE * 2 * v[0, 0, 0], rtol=1e-12)
    # unit inputs: norm on and off agree up to the epsilon
    L = 5
    q, k = _unit(_rand(rng, 1, L, 1, D)), _unit(_rand(rng, 1, L, 1, D))
    v, gl = _rand(rng, 1, L, 1, D), -rng.random((1, L, 1, D))
    beta = rng.random((1, L, 1))
    S0 = _rand(rng, 1, 1, D, D)
    args = (q, k, v, gl, beta, None, None, S0, [L], True)
    o_on, p_on = kio.infer_forward(*args, use_qk_l2norm=True)
    o_off, p_off = kio.infer_forward(*args, use_qk_l2norm=False)
    np.testing.assert_allclose(o_off, o_on, rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(p_off, p_on, rtol=1e-5, atol=1e-6)
    assert not np.array_equal(o_off, o_on)


def test_pool_slots_in_place_and_untouched():
    rng = np.random.default_rng(15)
    lengths, Hv = [3, 4, 2], 2
    T = sum(lengths)
    q, k = _rand(rng, 1, T, 1, D), _rand(rng, 1, T, 1, D)
    v, g = _rand(rng, 1, T, Hv, D), -rng.random((1, T, Hv, D))
    beta = rng.random((1, T, Hv))
    pool = _rand(rng, 6, Hv, D, D)
    idx = [4, 0, 2]
    o, new = kio.infer_forward(q, k, v, g, beta, None, None, pool, lengths, packed=True,
                               indices=idx)
    for s in (1, 3, 5):
        assert np.array_equal(new[s], pool[s])
    # each named slot equals a run with that slot as the initial state
    o2, fs2 = kio.infer_forward(q, k, v, g, beta, None, None, pool[idx], lengths, packed=True)
    assert np.array_equal(o, o2)
    for n, s in enumerate(idx):
        assert np.array_equal(new[s], fs2[n])
    with pytest.raises(ValueError):
        kio.infer_forward(q, k, v, g, beta, None, None, pool, lengths, packed=True, indices=[1, 1, 2])


def test_checkpoints_are_prefix_states():
    rng = np.random.default_rng(16)
    lengths, Hv, E = [5, 16, 17, 40], 2, 16
    T = sum(lengths)
    q, k = _rand(rng, 1, T, 1, D), _rand(rng, 1, T, 1, D)
    v, g = _rand(rng, 1, T, Hv, D), -rng.random((1, T, Hv, D))
    beta = rng.random((1, T, Hv))
    pool = _rand(rng, 4, Hv, D, D)
    o, new, ck = kio.infer_forward(q, k, v, g, beta, None, None, pool, lengths, packed=True,
                                   checkpoint_every=E)
    counts = [-(-L // E) for L in lengths]
    assert ck.shape[0] == sum(counts)
    row, t0 = 0, 0
    for n, L in enumerate(lengths):
        assert np.array_equal(ck[row], pool[n])
        for j in range(1, counts[n]):
            cut = j * E
            s = slice(t0, t0 + cut)
            _, fs = kio.infer_forward(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], None, None,
                                      pool[n:n + 1], [cut], packed=True)
            np.testing.assert_allclose(ck[row + j], fs[0], rtol=1e-12, atol=1e-12)
        row += counts[n]
        t0 += L


def test_spec_decode_slots_are_prefix_states():
    rng = np.random.default_rng(17)
    N, S, Hv = 3, 2, 2
    lengths = [1 + S] * N
    T = sum(lengths)
    q, k = _rand(rng, 1, T, 1, D), _rand(rng, 1, T, 1, D)
    v, g = _rand(rng, 1, T, Hv, D), -rng.random((1, T, Hv, D))
    beta = rng.random((1, T, Hv))
    pool = _rand(rng, 10, Hv, D, D)
    slots = [[4, 0, 7], [1, 9, 2], [3, 5, 6]]
    acc = [2, 0, 9]                         # clamped to 2, 1 and 3
    start_slot = [0, 1, 6]
    o, new = kio.infer_forward(q, k, v, g, beta, None, None, pool, lengths, packed=True,
                               indices=slots, num_spec_tokens=S, num_accepted=acc)
    assert np.array_equal(new[8], pool[8])   # named by no sequence
    for n in range(N):
        for t in range(1 + S):
            s = slice(n * (1 + S), n * (1 + S) + t + 1)
            o1, fs = kio.infer_forward(q[:, s], k[:, s], v[:, s], g[:, s], beta[:, s], None, None,
                                       pool[start_slot[n]:start_slot[n] + 1], [t + 1], packed=True)
            np.testing.assert_allclose(new[slots[n][t]], fs[0], rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(o[0, n * (1 + S) + t], o1[0, t], rtol=1e-12, atol=1e-12)


def test_source_pool_replaces_initial_state():
    rng = np.random.default_rng(18)
    lengths, Hv = [4, 6], 2
    T = sum(lengths)
    q, k = _rand(rng, 1, T, 1, D), _rand(rng, 1, T, 1, D)
    v, g = _rand(rng, 1, T, Hv, D), -rng.random((1, T, Hv, D))
    beta = rng.random((1, T, Hv))
    pool = _rand(rng, 3, Hv, D, D)
    src = _rand(rng, 2, Hv, D, D)
    src_copy = src.copy()
    o, new = kio.infer_forward(q, k, v, g, beta, None, None, pool, lengths, packed=True,
                               indices=[2, 0], source=src, source_indices=[1, 1])
    staged = pool.copy()
    staged[2], staged[0] = src[1], src[1]
    o2, new2 = kio.infer_forward(q, k, v, g, beta, None, None, staged, lengths, packed=True,
                                 indices=[2, 0])
    assert np.array_equal(o, o2) and np.array_equal(new[[0, 2]], new2[[0, 2]])
    assert np.array_equal(new[1], pool[1]) and np.array_equal(src, src_copy)
