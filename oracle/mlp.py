"""Gated-MLP intermediate activation Z, fp64 oracle (test infrastructure only).

Source: "In-Place Test-Time Training" as summarised on the iplexlaw.co.kr blog page
(arXiv 2604.06169, Feng et al.), section 2 (core principle 1): the transformer's gated MLP maps
its input through two projection paths, applies the gate, and forms the intermediate activation
Z that the final projection W_down (the fast weight) consumes.

Readings where the page is silent: the gate is SiLU (the gated MLP of the Qwen3 family the page
experiments with), Z = SiLU(X W_gate) * (X W_up) element by element, with W_gate and W_up
[d_model, d_ff] multiplying row vectors from the right, as the page writes its projections.
"""
from __future__ import annotations

import numpy as np

f64 = np.float64


def silu(x) -> np.ndarray:
    x = np.asarray(x, f64)
    return x / (1.0 + np.exp(-x))


def gated_z(X, W_gate, W_up) -> np.ndarray:
    """Z [T, d_ff] = SiLU(X W_gate) * (X W_up) for X [T, d_model]."""
    X = np.asarray(X, f64)
    return silu(X @ np.asarray(W_gate, f64)) * (X @ np.asarray(W_up, f64))


def gated_z_rows(X, W_gate, W_up, rows) -> np.ndarray:
    """Only the listed rows of Z (spot checks at large sizes)."""
    X = np.asarray(X)[list(rows)]
    return gated_z(X, W_gate, W_up)
