"""Plant plausible mistakes in the warm-up oracle (on the CPU); a pin must catch each."""
import numpy as np
import pytest

from oracle import warmup_oracle as W
import tests.test_warmup_oracle as P

_REAL_TARGET = W.dense_target
_REAL_KL = W.kl_and_grad


def _target_not_normalised(q, K, scale):
    return _REAL_TARGET(q, K, scale) * q.shape[0]         # plain sum over heads


def _target_without_scale(q, K, scale):
    return _REAL_TARGET(q, K, 1.0)


def _reversed_kl(a, I):
    m = I.max()
    logP = I - (m + np.log(np.exp(I - m).sum()))
    P = np.exp(logP)
    with np.errstate(divide="ignore"):
        loss = float(np.sum(P * (logP - np.log(a))))
    return loss, P - a


def _gradient_sign_flipped(a, I):
    loss, dI = _REAL_KL(a, I)
    return loss, -dI


def _relu_slope_one_at_zero(q, K, scale, qd, w, kd):
    a = W.dense_target(q, K, scale)
    z, I = W.indexer_parts(qd, w, kd)
    loss, dI = W.kl_and_grad(a, I)
    act = (z >= 0).astype(np.float64)
    coef = w[:, None] * act * dI[None, :]
    return loss, dI, np.maximum(z, 0.0) @ dI, coef @ kd, coef.T @ qd


def _dq_without_w(q, K, scale, qd, w, kd):
    a = W.dense_target(q, K, scale)
    z, I = W.indexer_parts(qd, w, kd)
    loss, dI = W.kl_and_grad(a, I)
    act = (z > 0).astype(np.float64)
    coef = w[:, None] * act * dI[None, :]
    return loss, dI, np.maximum(z, 0.0) @ dI, (act * dI[None, :]) @ kd, coef.T @ qd


def _dk_without_mask(q, K, scale, qd, w, kd):
    a = W.dense_target(q, K, scale)
    z, I = W.indexer_parts(qd, w, kd)
    loss, dI = W.kl_and_grad(a, I)
    act = (z > 0).astype(np.float64)
    coef = w[:, None] * act * dI[None, :]
    return loss, dI, np.maximum(z, 0.0) @ dI, coef @ kd, (w[:, None] * dI[None, :]).T @ qd


def _dk_overwritten_per_row(a, rows=None):
    """run_warmup with each row's key gradient replacing, not adding to, the earlier rows'."""
    T = a["q8"].shape[0]
    geo = W.row_geometry(a["seq_lens"], a["q_start"], T)
    rows = range(T) if rows is None else rows
    B, cap, d_I = a["k8"].shape
    H_I = a["q8"].shape[1]
    loss, dw = np.full(T, np.nan), np.zeros((T, H_I))
    dq, dk = np.zeros((T, H_I, d_I)), np.zeros((B, cap, d_I))
    for t in rows:
        b, p = geo[t]
        n = p + 1
        l, _, dwr, dqr, dkr = W.row_objective(a["q_f"][t], a["kv_f"][b, :n], float(a["scale"]),
                                              a["qd_f"][t], np.asarray(a["w"][t], dtype=np.float64),
                                              a["kd_f"][b, :n])
        loss[t], dw[t], dq[t] = l, dwr, dqr
        dk[b, :n] = dkr
    return {"loss": loss, "dI": {}, "dw": dw, "dq": dq, "dk": dk}


PINS = [P.test_target_is_head_mean_of_torch_softmax, P.test_one_head_target_is_that_heads_attention,
        P.test_kl_matches_scipy_entropy, P.test_perfect_indexer_has_zero_loss_and_gradient,
        P.test_single_token_row_is_exactly_zero, P.test_hand_worked_fixture_on_the_relu_kink,
        P.test_row_gradients_match_finite_differences, P.test_dI_matches_finite_differences_of_kl,
        P.test_batch_key_gradient_accumulates_over_rows]

MUTANTS = [
    ("dense_target", _target_not_normalised),
    ("dense_target", _target_without_scale),
    ("kl_and_grad", _reversed_kl),
    ("kl_and_grad", _gradient_sign_flipped),
    ("row_objective", _relu_slope_one_at_zero),
    ("row_objective", _dq_without_w),
    ("row_objective", _dk_without_mask),
    ("run_warmup", _dk_overwritten_per_row),
]


@pytest.mark.parametrize("fn_name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, fn_name, mutant):
    monkeypatch.setattr(W, fn_name, mutant)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            caught += 1
    assert caught >= 1, f"no pin noticed the planted mistake {mutant.__name__}"
