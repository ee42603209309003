"""In-Place TTT chunk scan, fp64 oracle (test infrastructure only).

Source: "In-Place Test-Time Training" as summarised on the iplexlaw.co.kr blog page
(arXiv 2604.06169, Feng et al.):

* section 2 (core principle 1): the gated MLP's final projection W_down is the fast weight; the
  chunk's output is its intermediate activation Z pushed through the current W_down, and the
  update is dW_down = eta * V_hat^T * Z.  Storage here follows that formula literally:
  W is [d_model, d_ff] (nn.Linear [out, in]) and a chunk's output is O_i = Z_i W_i^T.
* section 3 (core principle 2): apply-then-update.  Chunk i is produced from the state before
  its own update; the updated matrix is used from chunk i+1 on.
* section 4 (core principle 3): the target V_hat comes from a convolution of the token
  embeddings and W_target; the scan takes V_hat as an input.
* section 6 (context parallelism): the deltas are additive, so the state that chunk i sees is
  W_0 plus the exclusive prefix sum of the earlier deltas.

Readings where the page is silent: a last chunk shorter than ``chunk`` is allowed and is treated
like any other chunk; no norm clipping and no document-boundary reset are applied.
"""
from __future__ import annotations

import numpy as np

f64 = np.float64


def _as64(a) -> np.ndarray:
    return np.asarray(a).astype(f64, copy=False)


def chunk_scan(Z, V, W0, chunk: int, eta: float, block_rows: int = 0):
    """Sequential apply-then-update over one sequence (In-Place TTT page, sections 2-3).

    Z [T, d_ff], V [T, d_model] (V_hat), W0 [d_model, d_ff]; any float dtype, widened to fp64.
    Returns (O [T, d_model], W_final [d_model, d_ff]) in fp64.

    for each chunk i (rows [iC, min((i+1)C, T))):
        O_i  = Z_i W^T          # apply the state from before this chunk's update
        W   += eta V_i^T Z_i    # then update it for the following chunks
    """
    T = Z.shape[0]
    W = _as64(W0).copy()
    O = np.empty((T, W.shape[0]), f64)
    for i0 in range(0, T, chunk):
        i1 = min(T, i0 + chunk)
        Zi = _as64(Z[i0:i1])
        Vi = _as64(V[i0:i1])
        O[i0:i1] = Zi @ W.T
        W += eta * (Vi.T @ Zi)
    return O, W


def chunk_scan_batched(Z, V, W0, chunk: int, eta: float):
    """chunk_scan for each sequence of a batch: Z [B,T,d_ff], V [B,T,d_model],
    W0 [d_model,d_ff] (shared) or [B,d_model,d_ff]."""
    B = Z.shape[0]
    outs, ws = [], []
    for b in range(B):
        w0 = W0 if np.ndim(W0) == 2 else W0[b]
        o, w = chunk_scan(Z[b], V[b], w0, chunk, eta)
        outs.append(o)
        ws.append(w)
    return np.stack(outs), np.stack(ws)


def prefix_rows(Z, V, W0, chunk: int, eta: float, rows, block: int = 4096):
    """Selected output rows straight from the exclusive-prefix form (section 6).

    The state chunk i sees is W_0 + eta * sum_{j<i} V_j^T Z_j, so for a token t in chunk i
        O_t = W_0 z_t + eta * sum_{s < iC} (z_s . z_t) v_s.
    Exactly equal (up to rounding order) to the sequential scan; it lets a few rows of a very
    long sequence be checked without running the whole recurrence.  Returns [len(rows), d_model].
    """
    rows = np.asarray(rows, dtype=np.int64)
    Zr = _as64(Z[rows])
    out = Zr @ _as64(W0).T
    starts = (rows // chunk) * chunk          # first token of each row's own chunk
    smax = int(starts.max()) if rows.size else 0
    acc = np.zeros_like(out)
    for s0 in range(0, smax, block):
        s1 = min(smax, s0 + block)
        G = _as64(Z[s0:s1]) @ Zr.T                      # [s, rows]: z_s . z_t
        G *= (np.arange(s0, s1)[:, None] < starts[None, :])
        acc += G.T @ _as64(V[s0:s1])
    return out + eta * acc


def final_state_rows(Z, V, W0, eta: float, dm_rows, block: int = 4096):
    """Selected rows of the final state from additivity (section 6):
    W_final = W_0 + eta * sum_t v_t z_t^T, independent of the chunk size.
    Returns [len(dm_rows), d_ff]."""
    dm_rows = np.asarray(dm_rows, dtype=np.int64)
    T = Z.shape[0]
    acc = np.zeros((dm_rows.size, Z.shape[1]), f64)
    for s0 in range(0, T, block):
        s1 = min(T, s0 + block)
        acc += _as64(V[s0:s1][:, dm_rows]).T @ _as64(Z[s0:s1])
    return _as64(W0)[dm_rows] + eta * acc
