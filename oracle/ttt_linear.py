"""TTT-Linear mini-batch gradient descent, fp64 oracle (test infrastructure only).

Source: the TTT layers page ("AI that gets smarter while solving problems -- what is Test-Time
Training", ai-jitan-hub, on arXiv 2407.04620):

* section on making the hidden state a machine-learning model: the hidden state is itself a
  model and its update rule is one step of self-supervised learning; TTT-Linear's hidden state is
  a linear model.
* section on why test-time learning is not new: DeltaNet equals TTT-Linear with inner-loop
  mini-batch 1 and without LayerNorm and residual.
* In-Place TTT page, section 1.2: a typical TTT layer has a step that binds keys to values in
  the fast weight and a step that applies the *updated* fast weight to the query.

The mini-batch rule (one gradient step of 1/2 ||k W - v||^2 per mini-batch of b tokens, every
gradient taken at the start-of-mini-batch W, eta/b step) is the workload's fixed choice.  Reading
where the pages are silent: the query of token t sees the contributions of the tokens s <= t of
its own mini-batch (inclusive mask), which is what makes b = 1 the delta rule with the
post-update output.

Layouts: Q, K, V [T, H, dh] for one sequence; W [H, dh, dh] maps a row vector: o = q W.
"""
from __future__ import annotations

import numpy as np

f64 = np.float64


def _as64(a) -> np.ndarray:
    return np.asarray(a).astype(f64, copy=False)


def minibatch_gd(Q, K, V, W0, b: int, eta: float):
    """Dual-form mini-batch TTT-Linear over one sequence.

    For each head and each mini-batch m (rows [mb, (m+1)b)), with W the start-of-mini-batch state:
        R     = K_m W - V_m                       residual of the reconstruction loss
        loss_t = ||r_t||^2                        (by-product consumed by surprisal routing)
        O_m   = Q_m W - (eta/b) tril(Q_m K_m^T) R  output with the within-mini-batch updates
        W    <- W - (eta/b) K_m^T R                 one gradient step
    Returns (O [T,H,dh], W_final [H,dh,dh], loss [T,H]).
    """
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    T, H, dh = Q.shape
    if T % b:
        raise ValueError("T must be a multiple of the mini-batch size")
    W = np.zeros((H, dh, dh), f64) if W0 is None else _as64(W0).copy()
    O = np.empty((T, H, dh), f64)
    loss = np.empty((T, H), f64)
    lr = eta / b
    for h in range(H):
        Wh = W[h]
        for m0 in range(0, T, b):
            Km, Vm, Qm = K[m0:m0 + b, h], V[m0:m0 + b, h], Q[m0:m0 + b, h]
            R = Km @ Wh - Vm
            loss[m0:m0 + b, h] = np.sum(R * R, axis=1)
            A = np.tril(Qm @ Km.T)
            O[m0:m0 + b, h] = Qm @ Wh - lr * (A @ R)
            Wh = Wh - lr * (Km.T @ R)
        W[h] = Wh
    return O, W, loss


def minibatch_gd_batched(Q, K, V, W0, b: int, eta: float):
    """minibatch_gd for each sequence of Q, K, V [B,T,H,dh]; W0 [B,H,dh,dh] or None."""
    res = [minibatch_gd(Q[i], K[i], V[i], None if W0 is None else W0[i], b, eta)
           for i in range(Q.shape[0])]
    return tuple(np.stack(x) for x in zip(*res))


def delta_rule(Q, K, V, W0, eta: float):
    """Token-by-token delta rule (DeltaNet), the mini-batch-1 special case named on the TTT
    layers page: W <- W - eta k^T (k W - v); o_t = q_t W after token t's own update."""
    Q, K, V = _as64(Q), _as64(K), _as64(V)
    T, H, dh = Q.shape
    W = np.zeros((H, dh, dh), f64) if W0 is None else _as64(W0).copy()
    O = np.empty((T, H, dh), f64)
    for h in range(H):
        for t in range(T):
            k, v, q = K[t, h], V[t, h], Q[t, h]
            W[h] -= eta * np.outer(k, k @ W[h] - v)
            O[t, h] = q @ W[h]
    return O, W
