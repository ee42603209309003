"""LM-aligned target producer, fp64 oracle (test infrastructure only).

Source: "In-Place Test-Time Training" as summarised on the iplexlaw.co.kr blog page
(arXiv 2604.06169, Feng et al.):

* section 4 (core principle 3): the target is made from the token embeddings X0 by a 1-D
  convolution followed by a learnable projection, V_hat = Conv1D(X0) W_target; the kernel is
  arranged so that the target holds the next token, or several near-future tokens.
* section 6 (context parallelism): padding at chunk boundaries keeps the target's convolution
  from reading future information out of another chunk; the convolution is depthwise, and the
  long-context model used a kernel of size 5.

Readings where the page is silent: the convolution reads the `width` tokens after t, offsets
+1 .. +width (the near-future tokens; no current token), each channel with its own weight; a
token past the end of t's chunk (or past T) contributes zero. W_target multiplies from the
right, as written: V_hat = A W_target with W_target [d_in, d_out].
"""
from __future__ import annotations

import numpy as np

f64 = np.float64


def conv_rows(X0, conv_w, chunk: int) -> np.ndarray:
    """A[t] = sum_{j=1..width} conv_w[j-1] * X0[t+j], with X0 rows outside t's chunk taken as 0.

    X0 [T, d] and conv_w [width, d]; returns A [T, d] in fp64.
    """
    X0 = np.asarray(X0, f64)
    conv_w = np.asarray(conv_w, f64)
    T, d = X0.shape
    width = conv_w.shape[0]
    A = np.zeros((T, d), f64)
    for t in range(T):
        end = min((t // chunk + 1) * chunk, T)  # first token of the next chunk
        for j in range(1, width + 1):
            if t + j < end:
                A[t] += conv_w[j - 1] * X0[t + j]
    return A


def lm_target(X0, conv_w, W_target, chunk: int) -> np.ndarray:
    """V_hat = Conv1D(X0) W_target for one sequence: [T, d_in] x [d_in, d_out] -> [T, d_out]."""
    return conv_rows(X0, conv_w, chunk) @ np.asarray(W_target, f64)


def lm_target_batched(X0, conv_w, W_target, chunk: int) -> np.ndarray:
    """X0 [B, T, d_in]; the weights are shared by every sequence."""
    return np.stack([lm_target(x, conv_w, W_target, chunk) for x in np.asarray(X0)])


def lm_target_rows(X0, conv_w, W_target, chunk: int, rows) -> np.ndarray:
    """Only the listed rows of V_hat (each needs at most `width` rows of X0): for spot checks at
    sizes where the whole product would be slow."""
    X0 = np.asarray(X0)
    conv_w = np.asarray(conv_w, f64)
    W = np.asarray(W_target, f64)
    T = X0.shape[0]
    width = conv_w.shape[0]
    out = []
    for t in rows:
        end = min((t // chunk + 1) * chunk, T)
        a = np.zeros(X0.shape[1], f64)
        for j in range(1, width + 1):
            if t + j < end:
                a += conv_w[j - 1] * np.asarray(X0[t + j], f64)
        out.append(a @ W)
    return np.stack(out)
