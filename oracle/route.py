"""SR-TTT surprisal routing, step-by-step oracle (test infrastructure only).

Source: "SR-TTT: Surprisal-Aware Residual Test-Time Training" (gist.science technical summary,
arXiv 2603.06642):

* section 2.1, Surprisal Filter: the inner loop's forward pass yields a per-token reconstruction
  loss L_t; a token is routed when (1) L_t exceeds tau_EMA, an EMA-smoothed 95th-percentile
  threshold of recent losses, and (2) the mean loss of the token's local chunk is at least 80% of
  that threshold.
* section 2.1, Residual Cache: the keys and values of routed tokens go to a fixed-capacity
  cache that runs as a track of its own beside the fast weights.
* section 5: once saturated, the priority-based eviction behaves FIFO-like.

Readings where the page is silent (each is taken identically by the HIP path):

* L_t is the sum over heads of the per-head squared residual, accumulated in fp32 in head order
  h = 0, 1, ..., H-1.
* The percentile is nearest-rank: the k-th smallest of the chunk's n losses with
  k = ceil(pct * n) computed in fp64 and clamped to [1, n] (no interpolation).
* tau is per sequence; tau_0 = p_0, and before chunk c > 0 is routed
  tau_c = fl32(fl32(ema * tau_{c-1}) + fl32(w * p_c)) with w = fl32(1 - ema): two fp32 roundings,
  no fused multiply-add.
* The chunk mean is an fp64 pairwise sum of the chunk's fp32 losses -- padded with zeros to a power
  of two, adjacent pairs added level by level -- divided by n in fp64; condition 2 is
  mean >= fl64(f64(ratio) * f64(tau_c)).  Condition 1 is strict: L_t > tau_c in fp32.
* The cache is a FIFO ring: the r-th routed token of the sequence (token order, r from 0) goes to
  slot r mod capacity, so after the call the ring holds the newest `capacity` routed tokens.
  Empty slots hold index -1 and zero key/value rows.
"""
from __future__ import annotations

import math

import numpy as np

f32 = np.float32
f64 = np.float64


def head_sum(loss_th) -> np.ndarray:
    """L_t = sum_h loss[t, h], fp32 accumulation in head order. loss_th [T, H] -> [T] fp32."""
    loss_th = np.asarray(loss_th, dtype=f32)
    acc = np.zeros(loss_th.shape[0], f32)
    for h in range(loss_th.shape[1]):
        acc = (acc + loss_th[:, h]).astype(f32)
    return acc


def nearest_rank(values, pct: float):
    """k-th smallest value, k = ceil(pct * n) in fp64, clamped to [1, n]."""
    v = np.sort(np.asarray(values, dtype=f32))
    n = v.size
    k = min(max(int(math.ceil(f64(f32(pct)) * f64(n))), 1), n)
    return f32(v[k - 1])


def pairwise_sum_f64(values) -> f64:
    """Sum of fp32 values in fp64: zero-pad to a power of two, add adjacent pairs per level."""
    x = np.asarray(values, dtype=f32).astype(f64)
    m = 1
    while m < x.size:
        m *= 2
    x = np.concatenate([x, np.zeros(m - x.size, f64)])
    while x.size > 1:
        x = x[0::2] + x[1::2]
    return f64(x[0])


def ema_step(tau, p, ema: float):
    """tau' = fl32(fl32(ema*tau) + fl32(w*p)), w = fl32(1 - ema)."""
    e = f32(ema)
    w = f32(f32(1.0) - e)
    return f32(f32(e * f32(tau)) + f32(w * f32(p)))


def route_sequence(L, chunk: int, pct: float, ema: float, ratio: float):
    """Routing decisions for one sequence's per-token losses L [T] (fp32).

    Returns (tau [T/chunk] fp32, routed [T] bool)."""
    L = np.asarray(L, dtype=f32)
    T = L.size
    if T % chunk:
        raise ValueError("T must be a multiple of the routing chunk")
    nc = T // chunk
    taus = np.empty(nc, f32)
    routed = np.zeros(T, bool)
    tau = None
    for c in range(nc):
        Lc = L[c * chunk:(c + 1) * chunk]
        p = nearest_rank(Lc, pct)
        tau = p if c == 0 else ema_step(tau, p, ema)        # updated before routing chunk c
        taus[c] = tau
        mean = pairwise_sum_f64(Lc) / f64(chunk)
        ok = mean >= f64(f32(ratio)) * f64(tau)              # condition 2
        if ok:
            routed[c * chunk:(c + 1) * chunk] = Lc > tau     # condition 1 (strict)
    return taus, routed


def fifo_ring(routed, capacity: int):
    """Slots of a FIFO ring fed with the routed tokens in token order.

    Returns (slot_token [capacity] int32, -1 for empty, count, total)."""
    toks = np.flatnonzero(routed)
    total = int(toks.size)
    slots = np.full(capacity, -1, np.int32)
    for r, t in enumerate(toks):
        slots[r % capacity] = t
    return slots, min(total, capacity), total


def surprisal_route(loss, K, V, chunk: int, pct: float = 0.95, ema: float = 0.9,
                    ratio: float = 0.8, capacity: int = 256):
    """Whole routing step for a batch.

    loss [B,T,H] fp32; K, V [B,T,H*dh] (any dtype; rows are copied bit for bit).
    Returns a dict with tau [B,nc], mask [B,T] uint8, idx [B,cap] int32, k/v [B,cap,H*dh],
    count [B], total [B].
    """
    loss = np.asarray(loss, dtype=f32)
    B, T, H = loss.shape
    K = np.asarray(K).reshape(B, T, -1)
    V = np.asarray(V).reshape(B, T, -1)
    nc = T // chunk
    out = {
        "tau": np.empty((B, nc), f32), "mask": np.zeros((B, T), np.uint8),
        "idx": np.full((B, capacity), -1, np.int32),
        "k": np.zeros((B, capacity, K.shape[2]), K.dtype),
        "v": np.zeros((B, capacity, V.shape[2]), V.dtype),
        "count": np.zeros(B, np.int32), "total": np.zeros(B, np.int32),
    }
    for b in range(B):
        L = head_sum(loss[b])
        taus, routed = route_sequence(L, chunk, pct, ema, ratio)
        slots, count, total = fifo_ring(routed, capacity)
        out["tau"][b] = taus
        out["mask"][b] = routed.astype(np.uint8)
        out["idx"][b] = slots
        full = slots >= 0
        out["k"][b, full] = K[b, slots[full]]
        out["v"][b, full] = V[b, slots[full]]
        out["count"][b] = count
        out["total"][b] = total
    return out
