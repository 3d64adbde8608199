"""Pins of the warm-up objective oracle against things other than itself (CPU only).

The target is checked against torch.softmax, the KL against
scipy.stats.entropy, every gradient against central finite differences of
the oracle's own loss (which checks the hand-derived backward, not the
forward), the forward against closed forms (one token, a perfect indexer,
one head), and the whole chain against a hand-worked fixture that sits on
the ReLU kink.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.stats
import torch

import oracle
from oracle import warmup_oracle as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_row(rng, H=3, D=5, n=7, H_I=4, d_I=6):
    q = rng.standard_normal((H, D))
    K = rng.standard_normal((n, D))
    qd = rng.standard_normal((H_I, d_I))
    kd = rng.standard_normal((n, d_I))
    w = rng.standard_normal(H_I)
    return q, K, qd, w, kd


def test_target_is_head_mean_of_torch_softmax():
    rng = np.random.default_rng(1)
    q, K, *_ = _rand_row(rng, H=5, D=9, n=11)
    scale = 0.37
    got = W.dense_target(q, K, scale)
    logits = torch.from_numpy(scale * np.einsum("hd,sd->hs", q, K))
    ref = torch.softmax(logits, dim=1).mean(dim=0).numpy()
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-16)
    assert abs(got.sum() - 1.0) < 1e-14


def test_one_head_target_is_that_heads_attention():
    rng = np.random.default_rng(2)
    q, K, *_ = _rand_row(rng, H=1, D=4, n=6)
    x = 0.5 * (K @ q[0])
    ref = np.exp(x) / np.exp(x).sum()
    np.testing.assert_allclose(W.dense_target(q, K, 0.5), ref, rtol=1e-13)


def test_kl_matches_scipy_entropy():
    rng = np.random.default_rng(3)
    a = rng.random(9)
    a /= a.sum()
    a[3] = 0.0                          # a zero-probability target entry
    a /= a.sum()
    I = rng.standard_normal(9) * 3
    P = np.exp(I - I.max())
    P /= P.sum()
    loss, dI = W.kl_and_grad(a, I)
    assert loss == pytest.approx(scipy.stats.entropy(a, P), rel=1e-12, abs=1e-15)
    np.testing.assert_allclose(dI, P - a, atol=1e-15)


def test_perfect_indexer_has_zero_loss_and_gradient():
    rng = np.random.default_rng(4)
    a = rng.random(13)
    a /= a.sum()
    I = np.log(a) + 7.25                 # softmax(I) == a, whatever the shift
    loss, dI = W.kl_and_grad(a, I)
    assert abs(loss) < 1e-13
    assert np.abs(dI).max() < 1e-15


def test_single_token_row_is_exactly_zero():
    rng = np.random.default_rng(5)
    q, K, qd, w, kd = _rand_row(rng, n=1)
    loss, dI, dw, dqd, dkd = W.row_objective(q, K, 0.3, qd, w, kd)
    assert loss == 0.0
    assert np.all(dI == 0) and np.all(dw == 0) and np.all(dqd == 0) and np.all(dkd == 0)


def test_hand_worked_fixture_on_the_relu_kink():
    with open(os.path.join(GOLDEN, "warmup_hand.json")) as f:
        g = json.load(f)
    loss, dI, dw, dqd, dkd = W.row_objective(np.array(g["q"]), np.array(g["K"]), g["scale"],
                                             np.array(g["qd"]), np.array(g["w"]), np.array(g["kd"]))
    assert loss == pytest.approx(g["expected_loss"], rel=1e-14)
    np.testing.assert_allclose(dI, g["expected_dI"], rtol=1e-14)
    np.testing.assert_allclose(dw, g["expected_dw"], rtol=1e-14)
    np.testing.assert_allclose(dqd, g["expected_dqd"], rtol=1e-14, atol=1e-300)
    np.testing.assert_allclose(dkd, g["expected_dkd"], rtol=1e-14, atol=1e-300)
    # closed form of the fixture's loss
    assert g["expected_loss"] == pytest.approx(math.log(1 + math.e) - 0.5 - math.log(2), rel=1e-15)


def _fd(f, x, eps=1e-6):
    """Central finite differences of scalar f over every entry of x (modified in place)."""
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = x[i]
        x[i] = old + eps
        fp = f()
        x[i] = old - eps
        fm = f()
        x[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


def test_row_gradients_match_finite_differences():
    rng = np.random.default_rng(6)
    q, K, qd, w, kd = _rand_row(rng)
    z = qd @ kd.T
    assert np.abs(z).min() > 1e-3          # away from the kinks, where FD is valid
    scale = 0.4

    def loss():
        return W.row_objective(q, K, scale, qd, w, kd)[0]

    _, _, dw, dqd, dkd = W.row_objective(q, K, scale, qd, w, kd)
    np.testing.assert_allclose(dw, _fd(loss, w), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(dqd, _fd(loss, qd), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(dkd, _fd(loss, kd), rtol=1e-6, atol=1e-9)


def test_dI_matches_finite_differences_of_kl():
    rng = np.random.default_rng(7)
    a = rng.random(8)
    a /= a.sum()
    I = rng.standard_normal(8)
    _, dI = W.kl_and_grad(a, I)
    np.testing.assert_allclose(dI, _fd(lambda: W.kl_and_grad(a, I)[0], I), rtol=1e-6, atol=1e-10)


def _batch(rng, seq_lens=(5, 7), nq=(3, 7), H=2, D=4, H_I=3, d_I=5):
    B, cap = len(seq_lens), max(seq_lens) + 2
    q_start = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    T = int(q_start[-1])
    return {
        "q_f": rng.standard_normal((T, H, D)), "kv_f": rng.standard_normal((B, cap, D)),
        "scale": 0.6, "q8": np.zeros((T, H_I, d_I), np.uint8), "k8": np.zeros((B, cap, d_I), np.uint8),
        "qd_f": rng.standard_normal((T, H_I, d_I)), "kd_f": rng.standard_normal((B, cap, d_I)),
        "w": rng.standard_normal((T, H_I)), "seq_lens": np.array(seq_lens, np.int32), "q_start": q_start,
    }


def test_batch_key_gradient_accumulates_over_rows():
    """dk of the whole batch (keys shared by many rows) against FD of sum_t loss_t."""
    rng = np.random.default_rng(8)
    a = _batch(rng)
    res = W.run_warmup(a)

    def total():
        return float(np.sum(W.run_warmup(a)["loss"]))

    np.testing.assert_allclose(res["dk"], _fd(total, a["kd_f"]), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(res["dq"], _fd(total, a["qd_f"]), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(res["dw"], _fd(total, a["w"]), rtol=1e-6, atol=1e-9)
    # tokens past every sequence's length get nothing
    assert np.all(res["dk"][0, 5:] == 0) and np.all(res["dk"][1, 7:] == 0)


def test_rows_see_only_their_prefix():
    """Changing a token after a row's position changes neither that row's loss nor its dq."""
    rng = np.random.default_rng(9)
    a = _batch(rng, seq_lens=(6,), nq=(6,))
    r0 = W.run_warmup(a)
    a["kv_f"][0, 4] += 3.0
    a["kd_f"][0, 4] -= 2.0
    r1 = W.run_warmup(a)
    np.testing.assert_array_equal(r0["loss"][:4], r1["loss"][:4])
    np.testing.assert_array_equal(r0["dq"][:4], r1["dq"][:4])
    assert not np.allclose(r0["loss"][4:], r1["loss"][4:])


def test_fp8_inputs_decode_with_their_scales():
    """The FP8 route equals the float route fed the dequantised values."""
    rng = np.random.default_rng(10)
    a = _batch(rng, seq_lens=(5,), nq=(5,), H_I=2, d_I=4)
    codes = rng.integers(0, 256, size=a["q8"].shape).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                   # no NaN codes
    kcodes = rng.integers(0, 256, size=a["k8"].shape).astype(np.uint8)
    kcodes[(kcodes & 0x7F) == 0x7F] = 0x38
    a["q8"], a["k8"] = codes, kcodes
    a["q_scale"] = rng.random(5) + 0.5
    a["k_scale"] = rng.random((1, a["k8"].shape[1])) + 0.5
    fp8 = dict(a)
    fp8.pop("qd_f")
    fp8.pop("kd_f")
    r8 = W.run_warmup(fp8)
    a["qd_f"] = oracle.decode_e4m3fn(codes) * a["q_scale"][:, None, None]
    a["kd_f"] = oracle.decode_e4m3fn(kcodes) * a["k_scale"][:, :, None]
    rf = W.run_warmup(a)
    for name in ("loss", "dw", "dq", "dk"):
        np.testing.assert_array_equal(r8[name], rf[name])
