"""Seeded synthetic inputs at the shapes of the source pages' workloads.

Every tensor has its own seed and is drawn with numpy's PCG64 bit generator, so the same seed
gives the same bits on any machine. bf16 tensors are carried as uint16 bit patterns produced by
round-to-nearest-even from fp32; both the oracle (after widening to fp64) and the GPU library
consume exactly those bits.

Workload recipes (the pages measure on trained models and public evaluation suites that are not
available here; these synthetic draws take their shapes instead):

* In-Place TTT, small fp32 case: Z, V_hat ~ N(0, 1), W0 ~ N(0, 0.02^2).
* In-Place TTT at a Qwen3-4B-like MLP shape: Z = bf16(SiLU(X Wg) * (X Wu)) with X ~ N(0, 1) and
  Wg, Wu ~ N(0, 1/d_model); the target V_hat = bf16((sum_{j=1..4} c_j * X0_{t+j}) W_target), a
  depthwise causal-shifted kernel of width 4 over an independent draw X0 ~ N(0, 1), with rows past
  the end of the token's own chunk treated as zero, c ~ N(0, 1/4), W_target ~ N(0, 1/d_model);
  W0 ~ N(0, 1/d_ff). This is input synthesis only: the scan receives Z and V_hat as given.
* TTT-Linear multi-head: Q, K, V = bf16(X W_{Q,K,V}) with X ~ N(0, 1), W ~ N(0, 1/d_model).
* Surprisal routing: as TTT-Linear, except round(0.02 T) seeded positions per sequence whose X row
  is replaced by 8 g, g ~ N(0, I).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "bf16_round", "normal",
    "InplaceInputs", "inplace_f32", "inplace_mlp",
    "LinearInputs", "ttt_linear_inputs", "route_inputs",
]


# ----------------------------------------------------------------------------------------------
# bf16 packing (round to nearest, ties to even), done on the bit pattern of an fp32 value.
# ----------------------------------------------------------------------------------------------
def f32_to_bf16_bits(x) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even; NaNs stay quiet NaNs."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exact fp32 values they encode."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x) -> np.ndarray:
    """Round fp32 values to the nearest bf16 value, returned as fp32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))


def normal(seed: int, shape, std: float = 1.0) -> np.ndarray:
    """N(0, std^2) draw in fp32 from PCG64(seed)."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


# ----------------------------------------------------------------------------------------------
# In-Place TTT inputs.  Fast-weight layout: W is [d_model, d_ff] (nn.Linear [out, in] storage of
# the MLP down projection), so the update dW = eta * V_hat^T Z is stored as written on the page.
# ----------------------------------------------------------------------------------------------
@dataclass
class InplaceInputs:
    Z: np.ndarray        # [B, T, d_ff]   uint16 (bf16 bits) or float32
    V: np.ndarray        # [B, T, d_model] uint16 (bf16 bits) or float32
    W0: np.ndarray       # [d_model, d_ff] float32 (shared by all sequences) or [B, d_model, d_ff]
    chunk: int
    eta: float
    dtype: str           # "f32" or "bf16"
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, T, F = self.Z.shape
        return B, T, F, self.V.shape[2]

    def z_f64(self, b: int, rows=slice(None)) -> np.ndarray:
        z = self.Z[b, rows]
        return (bf16_bits_to_f32(z) if self.dtype == "bf16" else z).astype(np.float64)

    def v_f64(self, b: int, rows=slice(None)) -> np.ndarray:
        v = self.V[b, rows]
        return (bf16_bits_to_f32(v) if self.dtype == "bf16" else v).astype(np.float64)

    def w0_f64(self, b: int) -> np.ndarray:
        w = self.W0 if self.W0.ndim == 2 else self.W0[b]
        return w.astype(np.float64)


def inplace_f32(T: int, d_ff: int, d_model: int, chunk: int, eta: float, B: int = 1,
                seeds=(11, 12, 13), w_std: float = 0.02, shared_w0: bool = True) -> InplaceInputs:
    """Small fp32 In-Place case: Z, V_hat ~ N(0,1), W0 ~ N(0, w_std^2)."""
    Z = normal(seeds[0], (B, T, d_ff))
    V = normal(seeds[1], (B, T, d_model))
    W0 = normal(seeds[2], (d_model, d_ff) if shared_w0 else (B, d_model, d_ff), w_std)
    return InplaceInputs(Z, V, W0, chunk, eta, "f32", {"recipe": "normal", "seeds": seeds})


def _silu(x: np.ndarray) -> np.ndarray:
    return x / (np.float32(1.0) + np.exp(-x))


def inplace_mlp(T: int, d_model: int, d_ff: int, chunk: int, eta: float = 1e-4, B: int = 1,
                seed_base: int = 20, conv_width: int = 4, block: int = 4096,
                shared_w0: bool = True) -> InplaceInputs:
    """bf16 In-Place inputs from the gated-MLP recipe (seeds seed_base+1 .. seed_base+7).

    Sequence b > 0 uses seeds offset by 1000*b for its X and X0 draws; the projection weights,
    the target weights and W0 are shared.
    """
    s = seed_base
    Wg = normal(s + 2, (d_model, d_ff), 1.0 / math.sqrt(d_model))
    Wu = normal(s + 3, (d_model, d_ff), 1.0 / math.sqrt(d_model))
    cw = normal(s + 5, (conv_width, d_model), 0.5)
    Wt = normal(s + 6, (d_model, d_model), 1.0 / math.sqrt(d_model))
    W0 = normal(s + 7, (d_model, d_ff) if shared_w0 else (B, d_model, d_ff),
                1.0 / math.sqrt(d_ff))
    Z = np.empty((B, T, d_ff), np.uint16)
    V = np.empty((B, T, d_model), np.uint16)
    tok = np.arange(T)
    chunk_end = np.minimum((tok // chunk + 1) * chunk, T)
    for b in range(B):
        X = normal(s + 1 + 1000 * b, (T, d_model))
        X0 = normal(s + 4 + 1000 * b, (T, d_model))
        for r0 in range(0, T, block):
            r1 = min(T, r0 + block)
            xb = X[r0:r1]
            Z[b, r0:r1] = f32_to_bf16_bits(_silu(xb @ Wg) * (xb @ Wu))
            acc = np.zeros((r1 - r0, d_model), np.float32)
            for j in range(1, conv_width + 1):
                src = tok[r0:r1] + j
                ok = src < chunk_end[r0:r1]          # zero padding past the chunk's end
                rows = np.where(ok, src, 0)
                acc += np.where(ok[:, None], X0[rows], np.float32(0)) * cw[j - 1]
            V[b, r0:r1] = f32_to_bf16_bits(acc @ Wt)
    return InplaceInputs(Z, V, W0, chunk, eta, "bf16",
                         {"recipe": "gated-mlp", "seed_base": seed_base,
                          "conv_width": conv_width})


# ----------------------------------------------------------------------------------------------
# TTT-Linear / routing inputs: Q, K, V [B, T, H, dh] bf16 bits.
# ----------------------------------------------------------------------------------------------
@dataclass
class LinearInputs:
    Q: np.ndarray
    K: np.ndarray
    V: np.ndarray
    dtype: str
    meta: dict = field(default_factory=dict)

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return (bf16_bits_to_f32(a) if self.dtype == "bf16" else a).astype(np.float64)


def _project_heads(X: np.ndarray, seeds, H: int, dh: int, as_bf16: bool, block: int = 8192):
    B, T, dm = X.shape
    out = []
    for sd in seeds:
        Wp = normal(sd, (dm, H * dh), 1.0 / math.sqrt(dm))
        Y = np.empty((B, T, H, dh), np.uint16 if as_bf16 else np.float32)
        for b in range(B):
            for r0 in range(0, T, block):
                r1 = min(T, r0 + block)
                y = (X[b, r0:r1] @ Wp).reshape(r1 - r0, H, dh)
                Y[b, r0:r1] = f32_to_bf16_bits(y) if as_bf16 else y
        out.append(Y)
    return out


def ttt_linear_inputs(B: int, T: int, d_model: int, H: int, dh: int, seed_base: int = 40,
                      dtype: str = "bf16", qk_scale: float = 1.0) -> LinearInputs:
    """Q, K, V = X W_{Q,K,V}, X ~ N(0,1) (seed_base+1), W ~ N(0, 1/d_model) (seed_base+2..4).

    qk_scale multiplies X for the Q and K projections only (used to build small stable cases).
    """
    X = normal(seed_base + 1, (B, T, d_model))
    as_bf16 = dtype == "bf16"
    if qk_scale != 1.0:
        (V,) = _project_heads(X, (seed_base + 4,), H, dh, as_bf16)
        Q, K = _project_heads(X * np.float32(qk_scale), (seed_base + 2, seed_base + 3), H, dh,
                              as_bf16)
    else:
        Q, K, V = _project_heads(X, (seed_base + 2, seed_base + 3, seed_base + 4), H, dh,
                                 as_bf16)
    return LinearInputs(Q, K, V, dtype, {"seed_base": seed_base, "qk_scale": qk_scale})


def route_inputs(B: int = 4, T: int = 2048, d_model: int = 1024, H: int = 16, dh: int = 64,
                 seed_base: int = 50, outlier_frac: float = 0.02, outlier_scale: float = 8.0,
                 dtype: str = "bf16") -> LinearInputs:
    """Routing workload: N(0,1) tokens with round(outlier_frac*T) seeded outlier rows per sequence."""
    X = normal(seed_base + 1, (B, T, d_model))
    n_out = int(round(outlier_frac * T))
    g = np.random.Generator(np.random.PCG64(seed_base + 2))
    pos = np.stack([np.sort(g.choice(T, n_out, replace=False)) for _ in range(B)]) \
        if n_out > 0 else np.zeros((B, 0), np.int64)
    G = normal(seed_base + 3, (B, n_out, d_model))
    for b in range(B):
        X[b, pos[b]] = np.float32(outlier_scale) * G[b]
    Q, K, V = _project_heads(X, (seed_base + 4, seed_base + 5, seed_base + 6), H, dh,
                             dtype == "bf16")
    return LinearInputs(Q, K, V, dtype, {"seed_base": seed_base, "outliers": pos})
