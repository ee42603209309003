"""Pins of the reset/clip scan oracle (oracle/docs.py) against the plain scan oracle on the
pieces the page makes independent, and against facts of the mathematics."""
import numpy as np
import pytest

import oracle.docs as od
import oracle.inplace as oi


def _inputs(T=56, F=12, D=6, seed=0):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((T, F)), rng.standard_normal((T, D)), rng.standard_normal((D, F))


@pytest.mark.parametrize("start", [8, 16, 48])
def test_a_document_start_splits_the_sequence_into_independent_scans(start):
    Z, V, W0 = _inputs()
    O, W = od.chunk_scan_docs(Z, V, W0, 8, 0.05, [start])
    Op, _ = oi.chunk_scan(Z[:start], V[:start], W0, 8, 0.05)
    Os, Ws = oi.chunk_scan(Z[start:], V[start:], W0, 8, 0.05)
    np.testing.assert_allclose(O[:start], Op, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(O[start:], Os, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W, Ws, rtol=1e-12, atol=1e-12)


def test_no_document_and_no_clip_is_the_plain_scan_and_start_zero_is_a_no_op():
    Z, V, W0 = _inputs(T=53)
    O, W = oi.chunk_scan(Z, V, W0, 8, 0.05)
    for starts, tau in (((), None), ((0,), None), ((), 0.0), ((), float("inf")), ((0,), -1.0)):
        O2, W2 = od.chunk_scan_docs(Z, V, W0, 8, 0.05, starts, tau)
        np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(W2, W, rtol=1e-12, atol=1e-12)


def test_misaligned_document_start_is_rejected():
    Z, V, W0 = _inputs()
    with pytest.raises(ValueError):
        od.chunk_scan_docs(Z, V, W0, 8, 0.05, [12])


@pytest.mark.parametrize("tau", [1e-3, 0.05, 1.0, 1e3])
def test_a_clipped_delta_has_norm_min_of_its_norm_and_tau_and_keeps_its_direction(tau):
    # a one-chunk last document: W_final - W0 is exactly that chunk's clipped delta
    Z, V, W0 = _inputs(T=24)
    _, W = od.chunk_scan_docs(Z, V, W0, 8, 0.05, [16], tau)
    d = W - W0
    raw = 0.05 * (V[16:].T @ Z[16:])
    n = np.linalg.norm(raw)
    assert abs(np.linalg.norm(d) - min(n, tau)) <= 1e-12 * max(n, 1.0)
    cos = (d * raw).sum() / (np.linalg.norm(d) * n)
    assert abs(cos - 1.0) < 1e-12


def test_clipped_updates_do_not_depend_on_the_targets_scale():
    # with every delta clipped, scaling V scales no delta: outputs are unchanged
    Z, V, W0 = _inputs(seed=3)
    O1, W1 = od.chunk_scan_docs(Z, V, W0, 8, 0.05, [24], 1e-4)
    O2, W2 = od.chunk_scan_docs(Z, 7.0 * V, W0, 8, 0.05, [24], 1e-4)
    np.testing.assert_allclose(O2, O1, rtol=1e-10)
    np.testing.assert_allclose(W2, W1, rtol=1e-10)


def test_frobenius_norm_equals_the_gram_inner_product():
    # ||V^T Z||_F^2 = <Z Z^T, V V^T>_F: the identity a per-chunk norm pass can use instead of
    # forming the d_model x d_ff delta
    rng = np.random.default_rng(4)
    for T, F, D in ((5, 7, 3), (32, 40, 17)):
        Z, V = rng.standard_normal((T, F)), rng.standard_normal((T, D))
        lhs = np.linalg.norm(V.T @ Z) ** 2
        rhs = ((Z @ Z.T) * (V @ V.T)).sum()
        assert abs(lhs - rhs) <= 1e-11 * lhs
    n = od.delta_norms(Z, V, 8, 0.5)
    for i, i0 in enumerate(range(0, 32, 8)):
        zi, vi = Z[i0:i0 + 8], V[i0:i0 + 8]
        assert abs(n[i] - 0.5 * np.sqrt(((zi @ zi.T) * (vi @ vi.T)).sum())) <= 1e-12 * n[i]


def test_clip_scales_reproduce_the_clipped_scan_through_scaled_targets():
    # a clipped delta is the delta of targets scaled by the chunk's factor (the delta is linear
    # in V): the plain scan on scaled targets gives the clipped scan
    Z, V, W0 = _inputs(T=51, seed=5)
    tau = 0.3
    s = od.clip_scales(Z, V, 8, 0.05, tau)
    assert (s < 1).any() and (s <= 1).all()
    Vs = V * np.repeat(s, 8)[:51, None]
    O1, W1 = od.chunk_scan_docs(Z, V, W0, 8, 0.05, (), tau)
    O2, W2 = oi.chunk_scan(Z, Vs, W0, 8, 0.05)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(W1, W2, rtol=1e-12, atol=1e-12)


def test_planted_cumulative_clip_is_caught(monkeypatch):
    # clipping the accumulated change W - W0 instead of each delta disagrees with the per-delta
    # definition written out through the clip factors
    Z, V, W0 = _inputs(T=24)
    s = od.clip_scales(Z, V, 8, 0.05, 0.05)
    want = W0 + sum(s[i] * 0.05 * (V[8 * i:8 * i + 8].T @ Z[8 * i:8 * i + 8]) for i in range(3))
    _, W = od.chunk_scan_docs(Z, V, W0, 8, 0.05, (), 0.05)
    np.testing.assert_allclose(W, want, rtol=1e-12, atol=1e-12)

    def scan_cumulative(Z_, V_, W0_, chunk, eta, doc_starts=(), tau=None):
        W_ = np.asarray(W0_, float).copy()
        O_ = np.empty((Z_.shape[0], W_.shape[0]))
        for i0 in range(0, Z_.shape[0], chunk):
            O_[i0:i0 + chunk] = Z_[i0:i0 + chunk] @ W_.T
            W_ += eta * (V_[i0:i0 + chunk].T @ Z_[i0:i0 + chunk])
            W_ = W0_ + od.clip_factor(W_ - W0_, tau) * (W_ - W0_)
        return O_, W_

    monkeypatch.setattr(od, "chunk_scan_docs", scan_cumulative)
    _, Wbad = od.chunk_scan_docs(Z, V, W0, 8, 0.05, (), 0.05)
    assert not np.allclose(Wbad, want)


def test_gram_norms_match_the_explicit_delta_norms():
    Z, V, _ = _inputs(T=61, F=30, D=11, seed=12)
    np.testing.assert_allclose(od.delta_norms_gram(Z, V, 8, -0.3), od.delta_norms(Z, V, 8, -0.3),
                               rtol=1e-12)
