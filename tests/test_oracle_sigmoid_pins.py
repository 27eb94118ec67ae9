"""Pins of the oracle's sigmoid-bottleneck variant.

Paper: "Dual Dimensionality for Local and Global Attention", the paragraph
after Eq. (1): the authors also evaluated a sigmoid applied after the
down-projection, h^D = sigmoid(h W_down), and kept the linear form.  The
reading here is the logistic function 1 / (1 + e^-x) on each of the d_down
components, before the lift of Eq. (2).

Pins: hand values of the logistic function, the closed form at W_down = 0
(every component 1/2, so the lifted state is half the column sums of W_up and
the global keys at position 0, where RoPE is the identity, follow from it),
the symmetry sigmoid(-x) = 1 - sigmoid(x) under a negated W_down, and that
Eq. (2) lifts the activated latent (not the linear one).
"""
import numpy as np
import pytest

import dar_inputs as di
import oracle

# logistic function at -2, 0, 2 (1 / (1 + e^2), 1/2, 1 / (1 + e^-2))
SIG_M2, SIG_0, SIG_2 = 0.11920292202211755, 0.5, 0.8807970779778823


def _inp(B, N, d, H, d_k, d_down, seed):
    return di.prefill_inputs(B, N, d, H, d_k, d_down, dtype="f32", seed0=seed)


def _proj(x, H, d_k, act, pos0=0):
    return oracle.project(x["h"], x["W_down"], x["W_up"], x["W_Q"], x["W_K"], x["W_V"], H, d_k,
                          pos0=pos0, act=act)


def test_hand_values():
    d, d_down, H, d_k = 2, 3, 1, 2
    x = dict(h=np.array([[[1.0, 0.0]]]),
             W_down=np.array([[2.0, 0.0, -2.0], [5.0, 5.0, 5.0]]),
             W_up=np.eye(d_down, d), W_Q=np.zeros((d, H * d_k)), W_K=np.zeros((d, H * d_k)),
             W_V=np.zeros((d, H * d_k)))
    lin = _proj(x, H, d_k, "linear")["hD"][0, 0]
    sig = _proj(x, H, d_k, "sigmoid")["hD"][0, 0]
    assert np.array_equal(lin, [2.0, 0.0, -2.0])
    np.testing.assert_allclose(sig, [SIG_2, SIG_0, SIG_M2], rtol=0, atol=1e-15)
    # far tails: 1 and 0 within fp64
    x["W_down"] = np.array([[60.0, -60.0, 0.0], [0.0, 0.0, 0.0]])
    sig = _proj(x, H, d_k, "sigmoid")["hD"][0, 0]
    assert sig[0] == 1.0 and 0.0 <= sig[1] < 1e-25 and sig[2] == 0.5


def test_zero_down_projection_closed_form():
    B, N, d, H, d_k, d_down = 2, 5, 64, 2, 8, 16
    x = _inp(B, N, d, H, d_k, d_down, 8100)
    x["W_down"] = np.zeros_like(x["W_down"])
    P = _proj(x, H, d_k, "sigmoid")
    assert np.all(P["hD"] == 0.5)
    hp = 0.5 * x["W_up"].sum(axis=0)          # Eq. 2 with every latent component 1/2
    np.testing.assert_allclose(P["hp"], np.broadcast_to(hp, P["hp"].shape), rtol=1e-13,
                               atol=1e-13)
    for a in range(H):
        cols = slice(a * d_k, (a + 1) * d_k)
        # values carry no rotation: the same for every token
        np.testing.assert_allclose(P["VG"][:, a], np.broadcast_to(hp @ x["W_V"][:, cols],
                                                                  (B, N, d_k)), atol=1e-12)
        # keys at position 0, where the rotation is the identity
        np.testing.assert_allclose(P["KG"][:, a, 0], np.broadcast_to(hp @ x["W_K"][:, cols],
                                                                     (B, d_k)), atol=1e-12)
    # the local path and the queries do not see the bottleneck
    L = _proj(x, H, d_k, "linear")
    for k in ("Q", "KL", "VL"):
        assert np.array_equal(P[k], L[k])


def test_symmetry_under_negated_down_projection():
    B, N, d, H, d_k, d_down = 1, 7, 64, 1, 8, 32
    x = _inp(B, N, d, H, d_k, d_down, 8200)
    P = _proj(x, H, d_k, "sigmoid")
    x_neg = dict(x, W_down=-x["W_down"])
    Pn = _proj(x_neg, H, d_k, "sigmoid")
    np.testing.assert_allclose(P["hD"] + Pn["hD"], 1.0, rtol=0, atol=1e-15)
    assert np.all((P["hD"] > 0) & (P["hD"] < 1))
    # Eq. 2 is linear in the latent: the two lifts sum to the column sums of W_up
    np.testing.assert_allclose(P["hp"] + Pn["hp"],
                               np.broadcast_to(x["W_up"].sum(axis=0), P["hp"].shape),
                               rtol=1e-12, atol=1e-12)
    # a sign slip (1 / (1 + e^x)) would swap the two: the larger side follows h W_down
    lin = _proj(x, H, d_k, "linear")["hD"]
    assert np.array_equal(P["hD"] > 0.5, lin > 0)


def test_lift_uses_the_activated_latent():
    B, N, d, H, d_k, d_down = 1, 3, 64, 2, 8, 16
    x = _inp(B, N, d, H, d_k, d_down, 8300)
    P = _proj(x, H, d_k, "sigmoid", pos0=0)
    np.testing.assert_allclose(P["hp"], P["hD"] @ x["W_up"], rtol=1e-12, atol=1e-12)
    L = _proj(x, H, d_k, "linear", pos0=0)
    assert not np.allclose(P["KG"], L["KG"])


def test_rejects_unknown_activation():
    x = _inp(1, 1, 64, 1, 8, 16, 8400)
    with pytest.raises(ValueError):
        _proj(x, 1, 8, "tanh")
