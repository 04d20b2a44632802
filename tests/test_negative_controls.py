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


# ---------------------------------------------------------------------------
# inference oracle: mistakes in the option handling must fail its pins
# ---------------------------------------------------------------------------
from oracle import kda_infer_oracle as kio  # noqa: E402
import tests.test_infer_oracle_pins as ipins  # noqa: E402

INFER_PINS = [
    ipins.test_training_settings_reproduce_training_oracle,
    ipins.test_log_space_gate_closed_form_without_update,
    ipins.test_beta_as_given_stores_value_along_unit_key,
    ipins.test_norm_off_uses_keys_as_given,
    ipins.test_pool_slots_in_place_and_untouched,
    ipins.test_checkpoints_are_prefix_states,
    ipins.test_spec_decode_slots_are_prefix_states,
    ipins.test_source_pool_replaces_initial_state,
]


def _mut_infer_prologue(kind):
    real = kio.infer_prologue

    def bad(q, k, g, beta, A_log_h, dt_bias_h, use_qk_l2norm=True, use_gate_in_kernel=False,
            lower_bound=None, beta_is_logit=False, eps=ko.EPS):
        if kind == "gate_sign":              # exp(-g) for a log-space gate
            if not use_gate_in_kernel:
                g = -g
        elif kind == "beta_always_sigmoid":  # sigmoid applied to a given rate
            beta_is_logit = True
        elif kind == "norm_always_on":       # option ignored
            use_qk_l2norm = True
        elif kind == "log_gate_through_sigmoid":  # a log-space gate treated as raw input
            if not use_gate_in_kernel:
                use_gate_in_kernel, lower_bound = True, -5.0
                A_log_h, dt_bias_h = 0.0, None
        return real(q, k, g, beta, A_log_h, dt_bias_h, use_qk_l2norm, use_gate_in_kernel,
                    lower_bound, beta_is_logit, eps)
    return bad


def _caught(pins_list):
    failed = []
    for pin in pins_list:
        try:
            pin()
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("kind", ["gate_sign", "beta_always_sigmoid", "norm_always_on",
                                  "log_gate_through_sigmoid"])
def test_infer_option_mutant_is_caught(kind, monkeypatch):
    monkeypatch.setattr(kio, "infer_prologue", _mut_infer_prologue(kind))
    assert _caught(INFER_PINS), f"mutant {kind} passed every inference pin"


@pytest.mark.parametrize("kind", ["checkpoint_after_token", "spec_state_before_token",
                                  "spec_start_slot_zero"])
def test_infer_slot_mutant_is_caught(kind, monkeypatch):
    """Off-by-one mistakes in the checkpoint rows and the speculative slots."""
    real = ko.recurrence

    def rec(qn, kn, v, alpha, b, S0, scale=ko.SCALE, keep_states=False):
        o, S, states = real(qn, kn, v, alpha, b, S0, scale, keep_states=True)
        if kind in ("checkpoint_after_token", "spec_state_before_token"):
            # shift the state list by one token: rows/slots get a neighbour's state
            shift = 1 if kind == "checkpoint_after_token" else -1
            states = [states[min(max(i + shift, 0), len(states) - 1)] for i in range(len(states))]
        return (o, S, states) if keep_states else (o, S)
    if kind == "spec_start_slot_zero":
        real_fwd = kio.infer_forward

        def fwd(*a, **kw):
            if kw.get("num_spec_tokens"):
                kw["num_accepted"] = None     # ignore the accepted counts
            return real_fwd(*a, **kw)
        monkeypatch.setattr(kio, "infer_forward", fwd)
    else:
        monkeypatch.setattr(kio, "recurrence", rec)
    assert _caught(INFER_PINS), f"mutant {kind} passed every inference pin"
