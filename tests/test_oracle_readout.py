"""Pins of the residual-cache readout oracle (oracle/readout.py) against facts fixed by the page
and by the mathematics."""
import numpy as np
import pytest

import oracle.readout as orr
import oracle.route as oroute


def _inputs(B=2, T=64, H=2, dh=8, seed=0, density=0.3):
    rng = np.random.default_rng(seed)
    Q, K, V, O = (rng.standard_normal((B, T, H * dh)) for _ in range(4))
    routed = (rng.random((B, T)) < density).astype(np.uint8)
    alpha = rng.uniform(-0.5, 1.5, H * dh)
    return Q, K, V, O, routed, alpha


def test_no_routed_token_leaves_the_ttt_output_unchanged():
    Q, K, V, O, routed, alpha = _inputs()
    got = orr.cache_readout(Q, K, V, np.zeros_like(routed), O, alpha, 2, 8, 16, 0.3)
    np.testing.assert_array_equal(got, O)


def test_first_chunk_sees_an_empty_cache():
    Q, K, V, O, routed, alpha = _inputs()
    got = orr.cache_readout(Q, K, V, routed, O, alpha, 2, 16, 16, 0.3)
    np.testing.assert_array_equal(got[:, :16], O[:, :16])


def test_single_visible_entry_returns_its_value():
    # softmax over one logit is 1: the attention output is that entry's value row
    Q, K, V, O, _, _ = _inputs(B=1, T=16, H=2, dh=4)
    routed = np.zeros((1, 16), np.uint8)
    routed[0, 3] = 1
    alpha = np.ones(8)
    got = orr.cache_readout(Q, K, V, routed, O, alpha, 2, 8, 4, 0.5)
    np.testing.assert_allclose(got[0, 8:], O[0, 8:] + V[0, 3], rtol=1e-14, atol=1e-14)


def test_two_entries_follow_the_logistic_weights():
    rng = np.random.default_rng(3)
    dh = 4
    q, k1, k2, v1, v2 = (rng.standard_normal(dh) for _ in range(5))
    s1, s2 = 0.7 * q @ k1, 0.7 * q @ k2
    w1 = 1.0 / (1.0 + np.exp(s2 - s1))
    got = orr.attend(q, np.stack([k1, k2]), np.stack([v1, v2]), 0.7)
    np.testing.assert_allclose(got, w1 * v1 + (1 - w1) * v2, rtol=1e-13)


def test_equal_keys_average_the_values():
    rng = np.random.default_rng(4)
    k = rng.standard_normal(6)
    Vc = rng.standard_normal((5, 6))
    got = orr.attend(rng.standard_normal(6), np.tile(k, (5, 1)), Vc, 1.0)
    np.testing.assert_allclose(got, Vc.mean(axis=0), rtol=1e-13)


@pytest.mark.parametrize("a,expect", [(-0.3, 0.0), (0.0, 0.0), (0.25, 0.25), (1.0, 1.0), (3.0, 1.0)])
def test_alpha_is_clamped_to_the_unit_interval(a, expect):
    Q, K, V, O, routed, _ = _inputs(B=1, T=32, H=1, dh=4, seed=5, density=0.5)
    zero = np.zeros_like(O)
    full = orr.cache_readout(Q, K, V, routed, zero, np.ones(4), 1, 8, 8, 0.5)
    got = orr.cache_readout(Q, K, V, routed, O, np.full(4, a), 1, 8, 8, 0.5)
    np.testing.assert_allclose(got, O + expect * full, rtol=1e-13, atol=1e-13)


def test_chunk_never_reads_its_own_or_later_chunks():
    # changing every key, value and routing decision from chunk c on leaves outputs of chunks
    # <= c unchanged (their caches hold only earlier chunks' tokens)
    Q, K, V, O, routed, alpha = _inputs(B=1, T=64, seed=6, density=0.5)
    ref = orr.cache_readout(Q, K, V, routed, O, alpha, 2, 16, 8, 0.4)
    for c in range(4):
        K1, V1, r1 = K.copy(), V.copy(), routed.copy()
        K1[:, c * 16:] += 3.0
        V1[:, c * 16:] -= 2.0
        r1[:, c * 16:] = 1 - r1[:, c * 16:]
        got = orr.cache_readout(Q, K1, V1, r1, O, alpha, 2, 16, 8, 0.4)
        np.testing.assert_array_equal(got[:, :(c + 1) * 16], ref[:, :(c + 1) * 16])


def test_keys_and_values_of_unrouted_tokens_are_never_read():
    Q, K, V, O, routed, alpha = _inputs(seed=7)
    ref = orr.cache_readout(Q, K, V, routed, O, alpha, 2, 16, 8, 0.4)
    K1, V1 = K.copy(), V.copy()
    K1[routed == 0] = 1e3
    V1[routed == 0] = -1e3
    np.testing.assert_array_equal(orr.cache_readout(Q, K1, V1, routed, O, alpha, 2, 16, 8, 0.4), ref)


def test_eviction_keeps_the_newest_entries():
    # capacity 2, five tokens routed in chunk 0: chunk 1 sees only the last two. The evicted
    # ones get huge keys that would dominate the softmax if they were visible.
    T, dh = 16, 4
    rng = np.random.default_rng(8)
    Q = np.ones((1, T, dh))
    K = rng.standard_normal((1, T, dh)) * 0.1
    V = rng.standard_normal((1, T, dh))
    routed = np.zeros((1, T), np.uint8)
    routed[0, [0, 2, 3, 5, 7]] = 1
    K[0, [0, 2, 3]] = 50.0
    got = orr.cache_readout(Q, K, V, routed, np.zeros((1, T, dh)), np.ones(dh), 1, 8, 2, 1.0)
    want = orr.attend(Q[0, 8], K[0, [5, 7]], V[0, [5, 7]], 1.0)
    np.testing.assert_allclose(got[0, 8], want, rtol=1e-13)


def test_final_cache_matches_the_routing_oracles_ring():
    # the replayed cache after the last chunk holds exactly the routing oracle's ring entries
    rng = np.random.default_rng(9)
    for cap in (1, 3, 7, 64):
        routed = (rng.random(96) < 0.3).astype(np.uint8)
        states = orr.cache_states(routed, 16, cap)
        slots, count, _ = oroute.fifo_ring(routed, cap)
        assert sorted(states[-1]) == sorted(slots[slots >= 0].tolist())
        assert len(states[-1]) == count


def test_rows_sampler_matches_full_readout():
    Q, K, V, O, routed, alpha = _inputs(B=2, T=48, seed=10)
    full = orr.cache_readout(Q, K, V, routed, O, alpha, 2, 16, 5, 0.3)
    rows = [(0, 0), (0, 17), (1, 33), (1, 47)]
    got = orr.cache_readout_rows(Q, K, V, routed, O, alpha, 2, 16, 5, 0.3, rows)
    np.testing.assert_allclose(got, np.stack([full[b, t] for b, t in rows]), rtol=1e-13)


def test_planted_inclusive_cache_is_caught(monkeypatch):
    # a cache that already holds the token's own chunk (an inclusive reading) fails the
    # first-chunk pin
    Q, K, V, O, routed, alpha = _inputs(seed=11, density=0.6)

    def inclusive(routed_row, chunk, capacity):
        T = len(routed_row)
        return [list(np.flatnonzero(routed_row[:(c + 1) * chunk])[-capacity:])
                for c in range(T // chunk)] + [[]]

    monkeypatch.setattr(orr, "cache_states", inclusive)
    got = orr.cache_readout(Q, K, V, routed, O, alpha, 2, 16, 16, 0.3)
    assert not np.array_equal(got[:, :16], O[:, :16])
