"""Pins for the In-Place TTT oracle (CPU only).

Each check comes from something the source pages fix (In-Place TTT page, sections 2, 3 and 6),
from the mathematics, or from a hand-derived worked example -- never from the oracle itself.
"""
import json
import os

import numpy as np
import pytest

import oracle.inplace as oi

RNG = np.random.default_rng(7)


def _case(T=96, F=24, D=10, w_std=0.3):
    Z = RNG.standard_normal((T, F))
    V = RNG.standard_normal((T, D))
    W0 = RNG.standard_normal((D, F)) * w_std
    return Z, V, W0


def _mask(T, C):
    t = np.arange(T)
    return (t[None, :] // C) < (t[:, None] // C)       # M[t, s] = chunk(s) < chunk(t)


def test_hand_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "inplace_hand.json")))
    O, W = oi.chunk_scan(np.array(g["Z"], float), np.array(g["V"], float),
                         np.array(g["W0"], float), g["chunk"], g["eta"])
    np.testing.assert_array_equal(O, np.array(g["O"], float))
    np.testing.assert_array_equal(W, np.array(g["W_final"], float))


def test_eta_zero_gives_plain_projection():
    Z, V, W0 = _case()
    O, W = oi.chunk_scan(Z, V, W0, 16, 0.0)
    np.testing.assert_array_equal(W, W0)
    np.testing.assert_allclose(O, Z @ W0.T, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("C", [1, 7, 16, 32, 95, 96, 500])
def test_final_state_is_additive_for_every_chunk_size(C):
    Z, V, W0 = _case()
    eta = 0.05
    _, W = oi.chunk_scan(Z, V, W0, C, eta)
    np.testing.assert_allclose(W, W0 + eta * V.T @ Z, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C", [1, 5, 16, 40, 96, 200])
def test_quadratic_form(C):
    # Exclusive prefix (section 6): O = Z W0^T + eta (M o Z Z^T) V, M[t,s] = [chunk(s) < chunk(t)]
    Z, V, W0 = _case()
    eta = 0.03
    O, _ = oi.chunk_scan(Z, V, W0, C, eta)
    ref = Z @ W0.T + eta * (_mask(Z.shape[0], C) * (Z @ Z.T)) @ V
    np.testing.assert_allclose(O, ref, rtol=1e-11, atol=1e-11)


def test_causality_apply_then_update():
    # Section 3: chunk i's output never sees chunk i's own delta.
    Z, V, W0 = _case(T=64)
    C, eta = 16, 0.1
    O, _ = oi.chunk_scan(Z, V, W0, C, eta)
    for i in range(3):
        V2 = V.copy()
        V2[i * C:(i + 1) * C] += RNG.standard_normal((C, V.shape[1]))
        O2, _ = oi.chunk_scan(Z, V2, W0, C, eta)
        np.testing.assert_array_equal(O2[:(i + 1) * C], O[:(i + 1) * C])
        assert np.abs(O2[(i + 1) * C:(i + 2) * C] - O[(i + 1) * C:(i + 2) * C]).max() > 1e-6
    # changing z_t changes O_t and nothing else in chunks <= chunk(t)
    t = 21
    Z2 = Z.copy()
    Z2[t] += 1.0
    O2, _ = oi.chunk_scan(Z2, V, W0, C, eta)
    same = np.ones(64, bool)
    same[t] = False
    same[32:] = False
    np.testing.assert_array_equal(O2[same], O[same])
    assert np.abs(O2[t] - O[t]).max() > 1e-6


def test_chunk_at_least_T_and_zero_target():
    Z, V, W0 = _case()
    O, _ = oi.chunk_scan(Z, V, W0, Z.shape[0], 0.7)
    np.testing.assert_allclose(O, Z @ W0.T, rtol=1e-13, atol=1e-13)
    O, W = oi.chunk_scan(Z, np.zeros_like(V), W0, 8, 0.7)     # zero-initialised target
    np.testing.assert_allclose(O, Z @ W0.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(W, W0)


@pytest.mark.parametrize("T1", [32, 48, 80])
def test_resume_equals_single_call(T1):
    Z, V, W0 = _case()
    C, eta = 16, 0.02
    O, W = oi.chunk_scan(Z, V, W0, C, eta)
    Oa, Wa = oi.chunk_scan(Z[:T1], V[:T1], W0, C, eta)
    Ob, Wb = oi.chunk_scan(Z[T1:], V[T1:], Wa, C, eta)
    np.testing.assert_allclose(np.concatenate([Oa, Ob]), O, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Wb, W, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("C", [7, 16, 33])
def test_row_and_state_samplers_match_scan(C):
    Z, V, W0 = _case(T=150)
    eta = 0.04
    O, W = oi.chunk_scan(Z, V, W0, C, eta)
    rows = np.array([0, 5, C - 1, C, 2 * C + 3, 149])
    np.testing.assert_allclose(oi.prefix_rows(Z, V, W0, C, eta, rows, block=37), O[rows],
                               rtol=1e-11, atol=1e-11)
    dm = np.array([0, 3, 9])
    np.testing.assert_allclose(oi.final_state_rows(Z, V, W0, eta, dm, block=41), W[dm],
                               rtol=1e-11, atol=1e-11)


def test_batched_shared_and_per_sequence_state():
    B, T, F, D = 3, 40, 16, 8
    Z = RNG.standard_normal((B, T, F))
    V = RNG.standard_normal((B, T, D))
    W0 = RNG.standard_normal((D, F))
    O, W = oi.chunk_scan_batched(Z, V, W0, 8, 0.1)
    W0b = RNG.standard_normal((B, D, F))
    Ob, Wb = oi.chunk_scan_batched(Z, V, W0b, 8, 0.1)
    for b in range(B):
        o, w = oi.chunk_scan(Z[b], V[b], W0, 8, 0.1)
        np.testing.assert_array_equal(O[b], o)
        np.testing.assert_array_equal(W[b], w)
        o, w = oi.chunk_scan(Z[b], V[b], W0b[b], 8, 0.1)
        np.testing.assert_array_equal(Ob[b], o)


# ---- the pins must catch plausible mistakes planted in the oracle --------------------------
def _update_then_apply(Z, V, W0, chunk, eta):
    W = np.array(W0, float).copy()
    O = np.empty((Z.shape[0], W.shape[0]))
    for i0 in range(0, Z.shape[0], chunk):
        Zi, Vi = Z[i0:i0 + chunk], V[i0:i0 + chunk]
        W += eta * Vi.T @ Zi
        O[i0:i0 + chunk] = Zi @ W.T
    return O, W


def _sign_flip(Z, V, W0, chunk, eta):
    return _orig(Z, V, W0, chunk, -eta)


def _drop_ragged_update(Z, V, W0, chunk, eta):
    T = Z.shape[0]
    full = (T // chunk) * chunk
    O, W = _orig(Z, V, W0, chunk, eta)
    if full < T:
        W = W - eta * V[full:].T @ Z[full:]
    return O, W


_orig = oi.chunk_scan


def _pins_pass(golden_dir):
    try:
        test_hand_example(golden_dir)
        test_causality_apply_then_update()
        test_final_state_is_additive_for_every_chunk_size(7)
        test_quadratic_form(5)
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutant", [_update_then_apply, _sign_flip, _drop_ragged_update])
def test_planted_mistakes_are_caught(mutant, monkeypatch, golden_dir):
    assert _pins_pass(golden_dir)
    monkeypatch.setattr(oi, "chunk_scan", mutant)
    assert not _pins_pass(golden_dir)
