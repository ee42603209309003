"""In-Place TTT chunk scan with document-boundary reset and per-chunk update clipping, fp64
oracle (test infrastructure only).

Source: "In-Place Test-Time Training" as summarised on the iplexlaw.co.kr blog page
(arXiv 2604.06169, Feng et al.), section 6 (context parallelism) and its implementation notes:

* when an independent document ends, the fast weight goes back to its pre-trained state, so no
  information passes from one document to the next;
* for long contexts the Frobenius norm of each update delta is limited to a threshold (the page
  quotes 1e-5, from the paper's appendix C.2), which keeps the accumulated updates stable.

Readings where the page is silent:

* Documents start on chunk boundaries (token offsets that are multiples of the chunk); a chunk
  that begins a document is applied with W_0, and only the chunks of the same document before
  it contribute to the state later chunks see. W_final is the state after the last chunk, i.e.
  the last document's.
* The threshold is absolute and chosen by the caller: chunk i's delta dW_i = eta V_i^T Z_i is
  replaced by dW_i * min(1, tau / ||dW_i||_F); tau <= 0 or infinite means no clipping. (The
  page's 1e-5 may be relative to some norm; a caller wanting that passes the scaled value.)
* Apply-then-update order and storage are those of the plain scan: W is [d_model, d_ff],
  O_i = Z_i W^T.
"""
from __future__ import annotations

import math

import numpy as np

f64 = np.float64


def clip_factor(dW, tau) -> float:
    """min(1, tau / ||dW||_F); 1 when clipping is off or dW is zero."""
    if tau is None or not (tau > 0) or math.isinf(tau):
        return 1.0
    n = float(np.linalg.norm(dW))
    return 1.0 if n <= tau else tau / n


def chunk_scan_docs(Z, V, W0, chunk: int, eta: float, doc_starts=(), tau=None):
    """Sequential apply-then-update with resets at `doc_starts` and clipped deltas.

    Z [T, d_ff], V [T, d_model], W0 [d_model, d_ff]. Returns (O [T, d_model], W_final) in fp64.

    for each chunk i (rows [iC, min((i+1)C, T))):
        if a document starts at iC:  W = W0
        O_i = Z_i W^T
        dW  = eta V_i^T Z_i;   W += dW * min(1, tau / ||dW||_F)
    """
    Z = np.asarray(Z, f64)
    V = np.asarray(V, f64)
    W0 = np.asarray(W0, f64)
    T = Z.shape[0]
    starts = set(int(s) for s in doc_starts)
    for s in starts:
        if s % chunk or s < 0 or s >= max(T, 1) + chunk:
            raise ValueError("document starts must be chunk-aligned offsets inside the sequence")
    W = W0.copy()
    O = np.empty((T, W0.shape[0]), f64)
    for i0 in range(0, T, chunk):
        i1 = min(T, i0 + chunk)
        if i0 in starts:
            W = W0.copy()
        O[i0:i1] = Z[i0:i1] @ W.T
        dW = eta * (V[i0:i1].T @ Z[i0:i1])
        W += clip_factor(dW, tau) * dW
    return O, W


def delta_norms(Z, V, chunk: int, eta: float) -> np.ndarray:
    """||eta V_i^T Z_i||_F for every chunk, forming each delta explicitly."""
    Z = np.asarray(Z, f64)
    V = np.asarray(V, f64)
    return np.array([np.linalg.norm(eta * (V[i:i + chunk].T @ Z[i:i + chunk]))
                     for i in range(0, Z.shape[0], chunk)])


def clip_scales(Z, V, chunk: int, eta: float, tau) -> np.ndarray:
    """The factor each chunk's delta is multiplied by."""
    Z = np.asarray(Z, f64)
    V = np.asarray(V, f64)
    return np.array([clip_factor(eta * (V[i:i + chunk].T @ Z[i:i + chunk]), tau)
                     for i in range(0, Z.shape[0], chunk)])


def delta_norms_gram(Z, V, chunk: int, eta: float) -> np.ndarray:
    """||eta V_i^T Z_i||_F per chunk from the identity ||V^T Z||_F^2 = <Z Z^T, V V^T>_F (exact in
    exact arithmetic): C x C products instead of d_model x d_ff ones, for long sequences."""
    out = []
    for i in range(0, np.asarray(Z).shape[0], chunk):
        zi = np.asarray(Z[i:i + chunk], f64)
        vi = np.asarray(V[i:i + chunk], f64)
        out.append(abs(eta) * math.sqrt(max(((zi @ zi.T) * (vi @ vi.T)).sum(), 0.0)))
    return np.array(out)
