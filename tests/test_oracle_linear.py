"""Pins for the TTT-Linear oracle (CPU only): DeltaNet brute force at mini-batch 1 (TTT layers
page), the primal per-token form, causal linear attention as a closed form, and a hand example."""
import json
import os

import numpy as np
import pytest

import oracle.ttt_linear as ol

RNG = np.random.default_rng(11)


def _case(T=64, H=3, dh=8, qk_scale=0.35):
    Q = RNG.standard_normal((T, H, dh)) * qk_scale
    K = RNG.standard_normal((T, H, dh)) * qk_scale
    V = RNG.standard_normal((T, H, dh))
    W0 = RNG.standard_normal((H, dh, dh)) * 0.2
    return Q, K, V, W0


def test_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ttt_linear_hand.json")))
    arr = lambda k: np.array(g[k], float)
    O, W, loss = ol.minibatch_gd(arr("Q"), arr("K"), arr("V"), arr("W0"), g["b"], g["eta"])
    np.testing.assert_allclose(O, arr("O"), atol=1e-15)
    np.testing.assert_allclose(W, arr("W_final"), atol=1e-15)
    np.testing.assert_allclose(loss, arr("loss"), atol=1e-15)


@pytest.mark.parametrize("use_w0", [False, True])
def test_minibatch_one_is_the_delta_rule(use_w0):
    Q, K, V, W0 = _case()
    W0 = W0 if use_w0 else None
    eta = 0.5                       # eta * ||k||^2 < 2 keeps the delta rule stable here
    O, W, _ = ol.minibatch_gd(Q, K, V, W0, 1, eta)
    Od, Wd = ol.delta_rule(Q, K, V, W0, eta)
    np.testing.assert_allclose(O, Od, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W, Wd, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("b", [1, 4, 16, 64])
def test_dual_form_equals_primal_per_token_state(b):
    # Primal: token t in mini-batch m sees W_t = W_m - (eta/b) sum_{s in m, s<=t} k_s^T r_s,
    # with every residual r_s = k_s W_m - v_s taken at the start-of-mini-batch state.
    Q, K, V, W0 = _case()
    eta = 0.3
    O, W, loss = ol.minibatch_gd(Q, K, V, W0, b, eta)
    T, H, dh = Q.shape
    for h in range(H):
        Wm = W0[h].copy()
        for m0 in range(0, T, b):
            Wt = Wm.copy()
            grad = np.zeros_like(Wm)
            for t in range(m0, m0 + b):
                r = K[t, h] @ Wm - V[t, h]
                np.testing.assert_allclose(loss[t, h], r @ r, rtol=1e-12)
                Wt = Wt - (eta / b) * np.outer(K[t, h], r)
                grad += np.outer(K[t, h], r)
                np.testing.assert_allclose(O[t, h], Q[t, h] @ Wt, rtol=1e-11, atol=1e-11)
            Wm = Wm - (eta / b) * grad
        np.testing.assert_allclose(W[h], Wm, rtol=1e-11, atol=1e-11)


def test_zero_state_full_minibatch_is_causal_linear_attention():
    # W0 = 0 and b = T: o_t = (eta/T) sum_{s<=t} (q_t . k_s) v_s.
    Q, K, V, _ = _case(T=48)
    eta = 0.7
    T = Q.shape[0]
    O, W, _ = ol.minibatch_gd(Q, K, V, None, T, eta)
    for h in range(Q.shape[1]):
        S = np.tril(Q[:, h] @ K[:, h].T)
        np.testing.assert_allclose(O[:, h], (eta / T) * S @ V[:, h], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(W[h], (eta / T) * K[:, h].T @ V[:, h], rtol=1e-12,
                                   atol=1e-12)


def test_eta_zero_and_column_permutation():
    Q, K, V, W0 = _case()
    O, W, _ = ol.minibatch_gd(Q, K, V, W0, 16, 0.0)
    np.testing.assert_allclose(O, np.einsum("thd,hde->the", Q, W0), rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(W, W0)
    perm = RNG.permutation(Q.shape[2])
    O1, W1, _ = ol.minibatch_gd(Q, K, V, W0, 16, 0.4)
    O2, W2, _ = ol.minibatch_gd(Q, K, V[:, :, perm], W0[:, :, perm], 16, 0.4)
    np.testing.assert_allclose(O2, O1[:, :, perm], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W2, W1[:, :, perm], rtol=1e-12, atol=1e-12)


def test_first_minibatch_loss_closed_form():
    Q, K, V, W0 = _case()
    _, _, loss = ol.minibatch_gd(Q, K, V, W0, 16, 0.2)
    R = np.einsum("thd,hde->the", K[:16], W0) - V[:16]
    np.testing.assert_allclose(loss[:16], (R ** 2).sum(-1), rtol=1e-12)


def test_planted_exclusive_mask_is_caught(monkeypatch):
    # An exclusive within-mini-batch mask (s < t) breaks the delta-rule pin.
    real_tril = np.tril
    monkeypatch.setattr(ol.np, "tril", lambda a, k=0: real_tril(a, k - 1))
    with pytest.raises(AssertionError):
        test_minibatch_one_is_the_delta_rule(False)
