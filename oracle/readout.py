"""SR-TTT residual-cache readout with alpha fusion, fp64 oracle (test infrastructure only).

Source: "SR-TTT: Surprisal-Aware Residual Test-Time Training" (gist.science technical summary,
arXiv 2603.06642), section 2.1:

* Residual Cache: the keys and values of routed tokens are kept in a fixed-capacity cache that
  runs as a memory track of its own beside the fast weights.
* Alpha Fusion: the layer output is the TTT output plus a learned gate vector alpha times the
  attention output over the cache, Output = TTT(x) + alpha * CacheAttention(x); alpha is
  parameterised by a direct clamp instead of a sigmoid.
* section 5: once full, the cache's eviction behaves FIFO-like.

Readings where the page is silent:

* The cache a token reads is the cache as it stood when the token's routing chunk began: the
  routed tokens of earlier chunks, newest `capacity` of them (FIFO eviction), never tokens of
  the token's own or a later chunk (the same "before this chunk" rule as the fast weight).
* CacheAttention is per-head softmax attention of the token's query over the visible cached
  keys, with logits scale * (q . k), and the attention-weighted sum of the cached values; with
  no visible entry the attention output is zero.
* The clamp range of alpha is [0, 1] (a gate), applied per channel of the H * dh output.
"""
from __future__ import annotations

from collections import deque

import numpy as np

f64 = np.float64


def cache_states(routed_row, chunk: int, capacity: int):
    """The cache contents (token indices, oldest first) at the start of every chunk.

    The cache is replayed as the page describes it: tokens are offered in token order and a
    routed token enters the cache, evicting the oldest entry once `capacity` are held."""
    routed_row = np.asarray(routed_row)
    T = routed_row.shape[0]
    ring = deque()
    states = []
    for c in range(T // chunk):
        states.append(list(ring))
        for t in range(c * chunk, (c + 1) * chunk):
            if routed_row[t]:
                ring.append(t)
                if len(ring) > capacity:
                    ring.popleft()
    states.append(list(ring))  # after the last chunk: the cache the routing step leaves behind
    return states


def attend(q, Kc, Vc, scale: float) -> np.ndarray:
    """softmax_j(scale * q . k_j) weighted sum of v_j, fp64; zero for an empty cache."""
    if len(Kc) == 0:
        return np.zeros(np.asarray(Vc).shape[-1] if np.asarray(Vc).ndim == 2 else len(q), f64)
    s = scale * (np.asarray(Kc, f64) @ np.asarray(q, f64))
    w = np.exp(s - s.max())
    return (w / w.sum()) @ np.asarray(Vc, f64)


def cache_readout(Q, K, V, routed, ttt_out, alpha, H: int, chunk: int, capacity: int,
                  scale: float) -> np.ndarray:
    """Output [B, T, H*dh] = ttt_out + clamp(alpha, 0, 1) * CacheAttention.

    Q, K, V, ttt_out [B, T, H*dh]; routed [B, T] (nonzero = routed); alpha [H*dh]."""
    Q, K, V = (np.asarray(a, f64) for a in (Q, K, V))
    out = np.array(ttt_out, f64, copy=True)
    B, T, HD = Q.shape
    dh = HD // H
    gate = np.clip(np.asarray(alpha, f64), 0.0, 1.0)
    for b in range(B):
        states = cache_states(routed[b], chunk, capacity)
        for t in range(T):
            vis = states[t // chunk]
            if not vis:
                continue
            att = np.empty(HD, f64)
            for h in range(H):
                sl = slice(h * dh, (h + 1) * dh)
                att[sl] = attend(Q[b, t, sl], K[b, vis, sl], V[b, vis, sl], scale)
            out[b, t] += gate * att
    return out


def cache_readout_rows(Q, K, V, routed, ttt_out, alpha, H, chunk, capacity, scale, rows):
    """Only the listed (b, t) rows, for spot checks at large sizes."""
    Q, K, V = (np.asarray(a) for a in (Q, K, V))
    HD = Q.shape[2]
    dh = HD // H
    gate = np.clip(np.asarray(alpha, f64), 0.0, 1.0)
    res = []
    cache = {}
    for b, t in rows:
        if b not in cache:
            cache[b] = cache_states(routed[b], chunk, capacity)
        vis = cache[b][t // chunk]
        o = np.asarray(ttt_out[b, t], f64).copy()
        if vis:
            att = np.concatenate([attend(np.asarray(Q[b, t, h * dh:(h + 1) * dh], f64),
                                         np.asarray(K[b, vis, h * dh:(h + 1) * dh], f64),
                                         np.asarray(V[b, vis, h * dh:(h + 1) * dh], f64), scale)
                                  for h in range(H)])
            o += gate * att
        res.append(o)
    return np.stack(res)
