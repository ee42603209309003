"""Pins of the LM-aligned target oracle (oracle/target.py) against facts fixed by the page and by
the mathematics, not by the oracle itself."""
import numpy as np
import pytest

import gen
import oracle.target as ot

pytestmark = []


def _inputs(T=40, d=8, dout=6, width=4, seed=0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, d)), rng.standard_normal((width, d)),
            rng.standard_normal((d, dout)))


@pytest.mark.parametrize("chunk", [1, 5, 8, 13, 40, 100])
def test_no_row_of_a_later_chunk_is_read(chunk):
    # section 6: a chunk's targets never see the next chunk. Perturbing every row of chunks > i
    # leaves the targets of chunk i unchanged, for every i.
    X0, cw, W = _inputs()
    ref = ot.lm_target(X0, cw, W, chunk)
    T = X0.shape[0]
    for i in range(0, T, chunk):
        X1 = X0.copy()
        X1[i + chunk:] += 100.0
        got = ot.lm_target(X1, cw, W, chunk)
        np.testing.assert_array_equal(got[:i + chunk], ref[:i + chunk])


def test_width_one_unit_weight_is_next_token_projection():
    # a kernel reading only the next token with weight 1 gives V_hat_t = X0_{t+1} W_target, and
    # zero at the last token of every chunk (closed form)
    X0, _, W = _inputs(T=24)
    cw = np.ones((1, X0.shape[1]))
    got = ot.lm_target(X0, cw, W, 8)
    for t in range(24):
        want = np.zeros(W.shape[1]) if (t + 1) % 8 == 0 else X0[t + 1] @ W
        np.testing.assert_allclose(got[t], want, rtol=1e-13, atol=1e-13)


def test_zero_initialised_convolution_gives_zero_target():
    # the page initialises Conv1D to 0: the target starts at exactly zero
    X0, cw, W = _inputs()
    assert not ot.lm_target(X0, np.zeros_like(cw), W, 8).any()


def test_depthwise_channels_do_not_mix_before_the_projection():
    # with W_target = I, output channel c depends only on input channel c
    X0, cw, _ = _inputs()
    d = X0.shape[1]
    ref = ot.lm_target(X0, cw, np.eye(d), 7)
    X1 = X0.copy()
    X1[:, 3] += 5.0
    got = ot.lm_target(X1, cw, np.eye(d), 7)
    changed = np.flatnonzero(np.abs(got - ref).max(axis=0) > 0)
    assert changed.tolist() == [3]


def test_shifted_sum_matches_explicit_convolution():
    # inside one long chunk the depthwise convolution is numpy's correlation per channel
    X0, cw, W = _inputs(T=30, width=3)
    A = ot.conv_rows(X0, cw, 1000)
    for c in range(X0.shape[1]):
        full = np.correlate(np.concatenate([X0[1:, c], np.zeros(3)]), cw[:, c], mode="valid")
        np.testing.assert_allclose(A[:, c], full[:30], rtol=1e-12, atol=1e-12)


def test_matches_the_independent_generator_recipe():
    # gen.inplace_mlp builds V_hat for the scan's inputs with its own fp32 code: same
    # convolution (width 4, chunk-end zero padding) and projection. Recompute its V_hat from the
    # same seeds with the oracle; the only difference is fp32 accumulation and bf16 rounding.
    T, d, dff, C = 96, 32, 64, 32
    inp = gen.inplace_mlp(T, d, dff, C, eta=1e-3, seed_base=600)
    s = 600
    X0 = gen.normal(s + 4, (T, d))
    cw = gen.normal(s + 5, (4, d), 0.5)
    Wt = gen.normal(s + 6, (d, d), 1.0 / np.sqrt(d))
    ref = ot.lm_target(X0, cw, Wt, C)
    got = gen.bf16_bits_to_f32(inp.V[0]).astype(np.float64)
    err = np.abs(got - ref).max() / np.abs(ref).max()
    assert err < 1e-2, err


def test_rows_sampler_matches_full_product():
    X0, cw, W = _inputs(T=50)
    full = ot.lm_target(X0, cw, W, 9)
    rows = [0, 7, 8, 9, 26, 49]
    np.testing.assert_allclose(ot.lm_target_rows(X0, cw, W, 9, rows), full[rows], rtol=1e-12)


def test_planted_offset_mistake_is_caught(monkeypatch):
    # a convolution reading offsets 0..width-1 (the current token) fails the closed form
    X0, _, W = _inputs(T=16)
    cw = np.ones((1, X0.shape[1]))

    def wrong(X0_, conv_w, chunk):
        X0_ = np.asarray(X0_, np.float64)
        A = np.zeros_like(X0_)
        for t in range(X0_.shape[0]):
            A[t] += np.asarray(conv_w, np.float64)[0] * X0_[t]
        return A

    monkeypatch.setattr(ot, "conv_rows", wrong)
    got = ot.lm_target(X0, cw, W, 8)
    assert not np.allclose(got[0], X0[1] @ W)
