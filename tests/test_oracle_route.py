"""Pins for the surprisal-routing oracle (CPU only): hand-derived cases from the SR-TTT page's
rules, the nearest-rank percentile against numpy's inverted-CDF quantile, exact fp64 sums against
math.fsum, and the eta = 0 closed form of the loss."""
import json
import math
import os

import numpy as np
import pytest

import oracle.route as orr
import oracle.ttt_linear as ol

RNG = np.random.default_rng(5)


def _golden(golden_dir):
    return json.load(open(os.path.join(golden_dir, "route_hand.json")))


def test_hand_cases(golden_dir):
    g = _golden(golden_dir)
    p = g["params"]
    for c in g["cases"]:
        L = np.array(c["L"], np.float32)
        taus, routed = orr.route_sequence(L, c["chunk"], p["pct"], p["ema"], p["ratio"])
        assert np.flatnonzero(routed).tolist() == c["routed"], c["name"]
        if c["tau"] is not None:
            assert taus.tolist() == c["tau"], c["name"]
        slots, count, total = orr.fifo_ring(routed, c["capacity"])
        assert total == c["total"], c["name"]
        assert count == min(c["total"], c["capacity"])
        if "slots" in c:
            assert slots.tolist() == c["slots"], c["name"]


@pytest.mark.parametrize("n", [1, 2, 20, 63, 64, 100, 1000])
@pytest.mark.parametrize("pct", [0.05, 0.5, 0.95, 1.0])
def test_nearest_rank_matches_inverted_cdf_quantile(n, pct):
    x = RNG.standard_normal(n).astype(np.float32)
    ref = np.quantile(x.astype(np.float64), float(np.float32(pct)), method="inverted_cdf")
    assert orr.nearest_rank(x, pct) == np.float32(ref)


def test_pairwise_fp64_sum_is_exact_for_chunk_losses():
    for n in (1, 3, 64, 100, 1024):
        x = (RNG.random(n) * 1e3 + 1e-2).astype(np.float32)
        assert orr.pairwise_sum_f64(x) == math.fsum(x.astype(np.float64).tolist())


def test_head_sum_order_and_precision():
    loss = RNG.random((50, 16)).astype(np.float32)
    L = orr.head_sum(loss)
    assert L.dtype == np.float32
    np.testing.assert_allclose(L, loss.astype(np.float64).sum(1), rtol=1e-6)
    ref = np.float32(0)
    for h in range(16):
        ref = np.float32(ref + loss[7, h])
    assert L[7] == ref


def test_ema_of_constant_percentile_stays_put():
    for p in (1.0, 3.5, 1234.5, 1e-3):
        tau = np.float32(p)
        for _ in range(40):
            tau = orr.ema_step(tau, np.float32(p), 0.9)
        assert abs(tau - np.float32(p)) <= 4 * np.spacing(np.float32(p))


def test_route_conditions_hold_token_by_token():
    T, C = 2048, 64
    L = RNG.exponential(1.0, T).astype(np.float32)
    L[RNG.choice(T, 41, replace=False)] *= 64.0
    taus, routed = orr.route_sequence(L, C, 0.95, 0.9, 0.8)
    for c in range(T // C):
        Lc = L[c * C:(c + 1) * C]
        ok = math.fsum(Lc.astype(float)) / C >= float(np.float32(0.8)) * float(taus[c])
        for i in range(C):
            assert routed[c * C + i] == (ok and Lc[i] > taus[c])


def test_fifo_ring_keeps_newest_in_slot_order():
    routed = np.zeros(300, bool)
    routed[RNG.choice(300, 90, replace=False)] = True
    toks = np.flatnonzero(routed)
    slots, count, total = orr.fifo_ring(routed, 32)
    assert (total, count) == (90, 32)
    for r in range(90 - 32, 90):
        assert slots[r % 32] == toks[r]


def test_zero_step_loss_is_squared_value_norm():
    # eta = 0 and W0 = 0 keep W at zero, so L_t = sum_h ||v_{t,h}||^2 (closed form).
    T, H, dh = 128, 4, 8
    Q = RNG.standard_normal((T, H, dh))
    K = RNG.standard_normal((T, H, dh))
    V = RNG.standard_normal((T, H, dh)).astype(np.float32).astype(np.float64)
    _, _, loss = ol.minibatch_gd(Q, K, V, None, 64, 0.0)
    np.testing.assert_allclose(loss, (V ** 2).sum(-1), rtol=1e-15)
    out = orr.surprisal_route(loss[None].astype(np.float32), K[None], V[None], 64)
    assert out["total"][0] == out["mask"][0].sum()


def test_surprisal_route_copies_rows_and_marks_empty_slots():
    B, T, H, dh, C = 2, 256, 2, 4, 64
    loss = RNG.exponential(1.0, (B, T, H)).astype(np.float32)
    loss[0, 100] = 500.0
    loss[1, 10] = 800.0
    K = RNG.integers(0, 65535, (B, T, H * dh)).astype(np.uint16)
    V = RNG.integers(0, 65535, (B, T, H * dh)).astype(np.uint16)
    out = orr.surprisal_route(loss, K, V, C, capacity=8)
    for b in range(B):
        n = out["count"][b]
        idx = out["idx"][b]
        assert (idx[n:] == -1).all() or out["total"][b] > 8
        for s in range(8):
            if idx[s] >= 0:
                assert (out["k"][b, s] == K[b, idx[s]]).all()
                assert (out["v"][b, s] == V[b, idx[s]]).all()
            else:
                assert (out["k"][b, s] == 0).all()
    assert 100 in out["idx"][0] and 10 in out["idx"][1]


def test_planted_non_strict_compare_is_caught(golden_dir, monkeypatch):
    g = _golden(golden_dir)
    case = [c for c in g["cases"] if c["name"] == "ties_below_spikes"][0]
    real = orr.route_sequence

    def mutant(L, chunk, pct, ema, ratio):
        taus, routed = real(L, chunk, pct, ema, ratio)
        return taus, routed | (np.asarray(L) == np.repeat(taus, chunk))
    monkeypatch.setattr(orr, "route_sequence", mutant)
    with pytest.raises(AssertionError):
        test_hand_cases(golden_dir)
    assert case["routed"] == [61, 62, 63]
