"""Negative controls: plausible mistakes planted in the oracle (on the CPU) must
fail at least one pin. This shows the pins can tell the recurrence the pages
describe from its near neighbours."""
import numpy as np
import pytest

from oracle import kda_oracle as ko
import tests.test_oracle_pins as pins


def _mut_recurrence(kind):
    def rec(qn, kn, v, alpha, b, S0, scale=ko.SCALE, keep_states=False):
        S = S0.copy()
        L = qn.shape[0]
        o = np.empty((L, v.shape[1]))
        states = [S.copy()]
        for t in range(L):
            P = S * alpha[t][None, :]
            if kind == "readout_before_update":
                e = v[t] - P @ kn[t]
                o[t] = scale * (P @ qn[t])
                S = P + b[t] * np.outer(e, kn[t])
            elif kind == "decay_after_update":
                e = v[t] - S @ kn[t]
                S = (S + b[t] * np.outer(e, kn[t])) * alpha[t][None, :]
                o[t] = scale * (S @ qn[t])
            elif kind == "undecayed_error":
                e = v[t] - S @ kn[t]
                S = P + b[t] * np.outer(e, kn[t])
                o[t] = scale * (S @ qn[t])
            elif kind == "no_beta":
                e = v[t] - P @ kn[t]
                S = P + np.outer(e, kn[t])
                o[t] = scale * (S @ qn[t])
            elif kind == "transposed_readout":
                e = v[t] - P @ kn[t]
                S = P + b[t] * np.outer(e, kn[t])
                o[t] = scale * (S.T @ qn[t])
            elif kind == "error_sign":
                e = v[t] + P @ kn[t]
                S = P + b[t] * np.outer(e, kn[t])
                o[t] = scale * (S @ qn[t])
            elif kind == "row_decay":
                P = S * alpha[t][:, None]
                e = v[t] - P @ kn[t]
                S = P + b[t] * np.outer(e, kn[t])
                o[t] = scale * (S @ qn[t])
            else:
                raise KeyError(kind)
            states.append(S.copy())
        if keep_states:
            return o, S, states
        return o, S
    return rec


FORWARD_PINS = [
    pins.test_hand_worked_two_tokens,
    pins.test_single_token_from_zero_state,
    pins.test_beta_one_makes_state_recall_value,
    pins.test_beta_zero_is_pure_decay,
    pins.test_basis_keys_replace_columns,
]


@pytest.mark.parametrize("kind", ["readout_before_update", "decay_after_update",
                                  "undecayed_error", "no_beta", "transposed_readout",
                                  "error_sign", "row_decay"])
def test_forward_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(ko, "recurrence", _mut_recurrence(kind))
    failed = []
    for pin in FORWARD_PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {kind} passed every forward pin"


def _mut_backward(kind):
    real = ko.recurrence_backward

    def bwd(qn, kn, v, alpha, b, S0, do, dSL, scale=ko.SCALE, seg=64):
        dqn, dkn, dv, dalpha, db, dS0 = real(qn, kn, v, alpha, b, S0, do, dSL, scale, seg)
        if kind == "dk_drop_term":
            dkn = dkn * 0.999
        elif kind == "dalpha_sign":
            dalpha = -dalpha
        elif kind == "dS0_undecayed":
            dS0 = dS0 / alpha[0][None, :]
        elif kind == "dbeta_zero":
            db = db * 0.0
        return dqn, dkn, dv, dalpha, db, dS0
    return bwd


@pytest.mark.parametrize("kind", ["dk_drop_term", "dalpha_sign", "dS0_undecayed",
                                  "dbeta_zero"])
def test_backward_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(ko, "recurrence_backward", _mut_backward(kind))
    ok, info = pins._fd_check(11, 8, 11)
    assert not ok, f"mutant {kind} passed the finite-difference pin"


def test_prologue_eps_mutant_is_caught(monkeypatch):
    """A norm without its square root fails the library-routine pin."""
    real = ko.prologue

    def bad(q, k, g, beta, A_log_h, dt_bias_h, lb=ko.LOWER_BOUND, eps=ko.EPS):
        qn, kn, lam, alpha, b, z = real(q, k, g, beta, A_log_h, dt_bias_h, lb, eps)
        return qn * np.linalg.norm(q, axis=-1, keepdims=True) ** 0.01, kn, lam, alpha, b, z
    monkeypatch.setattr(ko, "prologue", bad)
    with pytest.raises(AssertionError):
        pins.test_prologue_matches_library_routines()
