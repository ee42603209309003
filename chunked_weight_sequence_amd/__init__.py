"""Chunked test-time-training fast-weight scan for MI355X (gfx950): Python binding.

A thin ctypes layer over ``libttt_mi355x.so`` (declared in ``include/ttt_mi355x.h``). It only
marshals arguments: PyTorch supplies device memory and the current HIP stream, and every step of
the computation runs in the library's HIP kernels. There is no fallback of any kind: if the
library is missing or the tensors are not on the GPU, the call raises.

    O, W = chunk_scan(Z, Vhat, W0, chunk=512, eta=1e-4)          # In-Place TTT
    O, W, loss = linear_minibatch(Q, K, V, minibatch=16, eta=0.1)  # TTT-Linear
    cache = surprisal_route(loss, K, V, chunk=64)                 # SR-TTT routing
    Vhat = lm_target(X0, conv_w, W_target, chunk=512)            # In-Place TTT target
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "lib", "library_path", "TTTError", "abi_version", "status_string",
    "chunk_scan", "chunk_scan_workspace_bytes", "chunk_scan_profile",
    "linear_minibatch", "surprisal_route", "lm_target", "gated_z", "cache_readout", "chunk_scan_docs",
    "chunk_scan_handover_timeouts", "scan_test_overrides", "chunk_scan_noalloc", "EXPORTED",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libttt_mi355x.so")

TTT_F32, TTT_BF16 = 0, 1
SCAN_PHASES = ("stage", "corr", "update", "apply")

# name -> (restype, argtypes); mirrors include/ttt_mi355x.h
_p, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_SCAN_ARGS = [_p, _p, _i, _p, _i, _p, _i, _p, _i, _i, _i, _i, _i, _f, _p, _sz, _p]
EXPORTED = {
    "ttt_chunk_scan": (_i, _SCAN_ARGS),
    "ttt_chunk_scan_workspace": (_sz, [_i, _i, _i, _i, _i, _i]),
    "ttt_chunk_scan_workspace_min": (_sz, [_i, _i, _i, _i, _i, _i]),
    "ttt_chunk_scan_noalloc": (_i, _SCAN_ARGS[:14] + [_p]),
    "ttt_chunk_scan_profile": (_i, _SCAN_ARGS + [_p, _p]),
    "ttt_chunk_scan_docs": (_i, _SCAN_ARGS[:14] + [_p, _p, _f] + _SCAN_ARGS[14:]),
    "ttt_chunk_scan_docs_workspace": (_sz, [_i, _i, _i, _i, _i, _i, _f]),
    "ttt_linear_minibatch": (_i, [_p, _p, _p, _i, _p, _p, _i, _p, _p,
                                  _i, _i, _i, _i, _i, _f, _p]),
    "ttt_surprisal_route": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _f, _f, _i,
                                 _p, _p, _p, _p, _p, _p, _p, _p]),
    "ttt_lm_target": (_i, [_p, _i, _p, _i, _p, _p, _i, _i, _i, _i, _i, _i, _p, _sz, _p]),
    "ttt_lm_target_workspace": (_sz, [_i, _i, _i, _i]),
    "ttt_gated_z": (_i, [_p, _i, _p, _p, _i, _i, _i, _i, _i, _p]),
    "ttt_cache_readout": (_i, [_p, _p, _p, _i, _p, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f,
                               _p]),
    "ttt_chunk_scan_handover_timeouts": (_i, [_i, _i, _i, _i, _i, _i, _p, _sz, _p, _p]),
    "ttt_scan_test_overrides": (_i, [_i, _i, _i]),
    "ttt_status_string": (ctypes.c_char_p, [_i]),
    "ttt_abi_version": (_i, []),
}

_lib = None


class TTTError(RuntimeError):
    """A non-OK status returned by the library."""


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(library_path):
            raise TTTError(f"{library_path} is missing: build it with "
                           "`python -m chunked_weight_sequence_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(library_path)
        for name, (res, args) in EXPORTED.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def abi_version() -> int:
    return lib().ttt_abi_version()


def status_string(code: int) -> str:
    return lib().ttt_status_string(code).decode()


def _check(code: int) -> None:
    if code != 0:
        raise TTTError(status_string(code))


# ---------------------------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    """Library dtype code of a tensor or a torch.dtype."""
    torch = _torch()
    dt = t if isinstance(t, torch.dtype) else t.dtype
    if dt == torch.float32:
        return TTT_F32
    if dt == torch.bfloat16:
        return TTT_BF16
    raise TypeError(f"unsupported dtype {dt}: use float32 or bfloat16")


def _dev(t, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _as3(t):
    return t if t.dim() == 3 else t.unsqueeze(0)


def chunk_scan_workspace_bytes(B, T, d_ff, d_model, chunk, dtype, minimum: bool = False) -> int:
    """Workspace bytes of chunk_scan for one pass, or (minimum=True) the least it accepts (bf16:
    segments of one group of chunks plus an fp32 state)."""
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    f = lib().ttt_chunk_scan_workspace_min if minimum else lib().ttt_chunk_scan_workspace
    return f(B, T, d_ff, d_model, chunk, code)


def _need(t, name: str, shape, dtype, device):
    """Checks that an output tensor passed in by the caller has exactly the shape, dtype and
    device the kernels will write (the C ABI sees only its pointer)."""
    _dev(t, name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    return t


def _scan_prepare(Z, Vhat, W0, chunk, eta, out_dtype, O, W_final, workspace, final_state):
    torch = _torch()
    Z3, V3 = _dev(_as3(Z), "Z"), _dev(_as3(Vhat), "Vhat")
    B, T, F = Z3.shape
    D = V3.shape[2]
    dev = Z3.device
    if V3.shape[:2] != (B, T):
        raise ValueError("Z and Vhat must agree on [B, T]")
    if V3.dtype != Z3.dtype:
        raise TypeError(f"Vhat must have Z's dtype {Z3.dtype}, got {V3.dtype}")
    if V3.device != dev:
        raise ValueError("Z and Vhat must be on one device")
    _dev(W0, "W0")
    if W0.dtype != torch.float32:
        raise TypeError("W0 must be float32")
    if W0.device != dev:
        raise ValueError("W0 must be on Z's device")
    if tuple(W0.shape) == (D, F):
        shared = 1
    elif tuple(W0.shape) == (B, D, F):
        shared = 0
    else:
        raise ValueError(f"W0 must be [d_model, d_ff] = [{D}, {F}] or [B, d_model, d_ff] = "
                         f"[{B}, {D}, {F}], got {tuple(W0.shape)}")
    out_dtype = out_dtype or Z3.dtype
    if O is None:
        O = torch.empty((B, T, D), dtype=out_dtype, device=dev)
    else:
        O = _as3(O)
        _need(O, "O", (B, T, D), None, dev)
        _dtype_code(O)
    if W_final is None and final_state:
        W_final = torch.empty((B, D, F), dtype=torch.float32, device=dev)
    if W_final is not None:
        # [B, d_model, d_ff], or [d_model, d_ff] for a single sequence (e.g. W0 itself)
        want = (D, F) if (W_final.dim() == 2 and B == 1) else (B, D, F)
        _need(W_final, "W_final", want, torch.float32, dev)
    code = _dtype_code(Z3)
    need = lib().ttt_chunk_scan_workspace(B, T, F, D, chunk, code)
    if workspace is False:       # the caller sizes its own workspace
        workspace = None
    elif workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        _dev(workspace, "workspace")
        if workspace.device != dev:
            raise ValueError("workspace must be on Z's device")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = [_ptr(Z3), _ptr(V3), code, _ptr(W0), shared, _ptr(O), _dtype_code(O),
            _ptr(W_final), B, T, F, D, chunk, float(eta), _ptr(workspace),
            ws_bytes, _stream(Z3)]
    return args, O, W_final


def chunk_scan(Z, Vhat, W0, chunk: int, eta: float, *, out_dtype=None, O=None, W_final=None,
               workspace=None, final_state: bool = True):
    """In-Place TTT scan. Z [B,T,d_ff] or [T,d_ff], Vhat [B,T,d_model] (same dtype), W0
    [d_model,d_ff] fp32 (shared) or [B,d_model,d_ff]. Returns (O [B,T,d_model], W_final
    [B,d_model,d_ff] or None)."""
    args, O, W_final = _scan_prepare(Z, Vhat, W0, chunk, eta, out_dtype, O, W_final, workspace,
                                     final_state)
    _check(lib().ttt_chunk_scan(*args))
    return O, W_final


def chunk_scan_noalloc(Z, Vhat, W0, chunk: int, eta: float, *, O, W_final=None):
    """ttt_chunk_scan_noalloc: the scan with its workspace taken from the library's static device
    scratch (no allocation by the library; O and W_final are the caller's). Returns (O, W_final)."""
    args, O, W_final = _scan_prepare(Z, Vhat, W0, chunk, eta, None, O, W_final, False, False)
    _check(lib().ttt_chunk_scan_noalloc(*(args[:14] + [args[16]])))
    return O, W_final


def chunk_scan_docs(Z, Vhat, W0, chunk: int, eta: float, *, doc_starts=None, clip_tau=0.0,
                    out_dtype=None, O=None, W_final=None, workspace=None,
                    final_state: bool = True):
    """chunk_scan with document-boundary resets and per-chunk update clipping. doc_starts: None
    or one list per sequence of chunk-aligned token offsets in (0, T) where a new document
    begins; clip_tau: absolute Frobenius threshold per chunk delta (<= 0: off). Returns
    (O, W_final)."""
    args, O, W_final = _scan_prepare(Z, Vhat, W0, chunk, eta, out_dtype, O, W_final, False,
                                     final_state)
    B, T, F, D, code = args[8], args[9], args[10], args[11], args[2]
    torch = _torch()
    need = lib().ttt_chunk_scan_docs_workspace(B, T, F, D, chunk, code, float(clip_tau))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=O.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    counts = starts = None
    if doc_starts is not None:
        if len(doc_starts) != B:
            raise ValueError("doc_starts needs one list per sequence")
        flat = [int(x) for d in doc_starts for x in d]
        counts = (ctypes.c_int * B)(*[len(d) for d in doc_starts])
        starts = (ctypes.c_int * max(1, len(flat)))(*flat)
    args = args[:14] + [None if starts is None else ctypes.addressof(starts),
                        None if counts is None else ctypes.addressof(counts), float(clip_tau),
                        _ptr(workspace), ws_bytes, args[16]]
    _check(lib().ttt_chunk_scan_docs(*args))
    return O, W_final


def chunk_scan_handover_timeouts(workspace, B, T, d_ff, d_model, chunk, dtype):
    """How many state-chain hand-over waits ran out (and were recomputed) in the last scan call
    that used `workspace` with these sizes: a device int32 tensor of one element, written on the
    current stream (no synchronisation)."""
    torch = _torch()
    _dev(workspace, "workspace")
    count = torch.empty(4, dtype=torch.int32, device=workspace.device)
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    _check(lib().ttt_chunk_scan_handover_timeouts(
        B, T, d_ff, d_model, chunk, code, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(count), _stream(workspace)))
    return count[:1]


def scan_test_overrides(group_tokens: int = 0, token_split: int = -1, spin_limit: int = -1):
    """FOR TESTS ONLY: process-wide schedule overrides of the bf16 scan (see the header);
    scan_test_overrides() restores the defaults."""
    _check(lib().ttt_scan_test_overrides(int(group_tokens), int(token_split), int(spin_limit)))


def chunk_scan_profile(Z, Vhat, W0, chunk: int, eta: float, *, out_dtype=None, O=None,
                       W_final=None, workspace=None, final_state: bool = True):
    """chunk_scan with per-phase HIP-event timing; synchronises. Returns (O, W_final, {phase:
    (ms, launches)})."""
    args, O, W_final = _scan_prepare(Z, Vhat, W0, chunk, eta, out_dtype, O, W_final, workspace,
                                     final_state)
    ms = (ctypes.c_float * 4)()
    n = (ctypes.c_int * 4)()
    _check(lib().ttt_chunk_scan_profile(*args, ctypes.addressof(ms), ctypes.addressof(n)))
    return O, W_final, {p: (ms[i], n[i]) for i, p in enumerate(SCAN_PHASES)}


def linear_minibatch(Q, K, V, minibatch: int, eta: float, *, W0=None, out_dtype=None,
                     with_loss: bool = True, final_state: bool = True, O=None, W_final=None,
                     loss=None):
    """TTT-Linear mini-batch GD. Q, K, V [B,T,H,dh]; W0 [B,H,dh,dh] fp32 or None (zeros).
    Returns (O [B,T,H,dh], W_final [B,H,dh,dh] or None, loss [B,T,H] or None)."""
    torch = _torch()
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _dev(t, n)
    if not (Q.shape == K.shape == V.shape) or Q.dim() != 4:
        raise ValueError("Q, K, V must share one [B, T, H, dh] shape")
    if not (Q.dtype == K.dtype == V.dtype):
        raise TypeError("Q, K, V must share one dtype")
    B, T, H, dh = Q.shape
    dev = Q.device
    if W0 is not None:
        _dev(W0, "W0")
        if W0.dtype != torch.float32 or tuple(W0.shape) != (B, H, dh, dh):
            raise ValueError("W0 must be float32 [B, H, dh, dh]")
    for t, n in ((K, "K"), (V, "V")):
        if t.device != dev:
            raise ValueError(f"{n} must be on Q's device")
    if W0 is not None and W0.device != dev:
        raise ValueError("W0 must be on Q's device")
    if O is None:
        O = torch.empty((B, T, H, dh), dtype=out_dtype or Q.dtype, device=dev)
    else:
        _need(O, "O", (B, T, H, dh), out_dtype, dev)
        _dtype_code(O)
    if W_final is None and final_state:
        W_final = torch.empty((B, H, dh, dh), dtype=torch.float32, device=dev)
    elif W_final is not None:
        _need(W_final, "W_final", (B, H, dh, dh), torch.float32, dev)
    if loss is None and with_loss:
        loss = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    elif loss is not None:
        _need(loss, "loss", (B, T, H), torch.float32, dev)
    _check(lib().ttt_linear_minibatch(_ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), _ptr(W0),
                                      _ptr(O), _dtype_code(O), _ptr(W_final), _ptr(loss),
                                      B, T, H, dh, minibatch, float(eta), _stream(Q)))
    return O, W_final, loss


def surprisal_route(loss, K, V, chunk: int, *, pct: float = 0.95, ema: float = 0.9,
                    ratio: float = 0.8, capacity: int = 256, want_kv: bool = True,
                    want_mask: bool = True, out: dict | None = None):
    """SR-TTT routing. loss [B,T,H] fp32; K, V [B,T,H,dh] or [B,T,H*dh]. Returns a dict with
    tau [B,T/chunk], mask [B,T] uint8, idx [B,cap] int32, k/v [B,cap,H*dh], count [B],
    total [B]. `out` may pass that dict back in to reuse its tensors (same shapes)."""
    torch = _torch()
    _dev(loss, "loss")
    if loss.dtype != torch.float32 or loss.dim() != 3:
        raise ValueError("loss must be float32 [B, T, H]")
    B, T, H = loss.shape
    _dev(K, "K")
    _dev(V, "V")
    dev = loss.device
    if K.dim() < 3 or tuple(K.shape[:2]) != (B, T) or K.shape != V.shape or K.dtype != V.dtype:
        raise ValueError("K and V must share one [B, T, H, dh] or [B, T, H*dh] shape and dtype, "
                         "with loss's B and T")
    if K.device != dev or V.device != dev:
        raise ValueError("K and V must be on loss's device")
    row = K[0, 0].numel()
    if row % H:
        raise ValueError("K rows must hold H * dh elements")
    dh = row // H
    if out is not None:
        torch_i32, torch_f32 = torch.int32, torch.float32
        want = {"tau": ((B, T // chunk), torch_f32), "idx": ((B, capacity), torch_i32),
                "count": ((B,), torch_i32), "total": ((B,), torch_i32)}
        for name, (shape, dt) in want.items():
            _need(out[name], f"out[{name!r}]", shape, dt, dev)
        for name in ("k", "v"):
            if out.get(name) is not None:
                _need(out[name], f"out[{name!r}]", (B, capacity, row), K.dtype, dev)
        if out.get("mask") is not None:
            _need(out["mask"], "out['mask']", (B, T), torch.uint8, dev)
    else:
        out = {
        "tau": torch.empty((B, T // chunk), dtype=torch.float32, device=dev),
        "mask": torch.empty((B, T), dtype=torch.uint8, device=dev) if want_mask else None,
        "idx": torch.empty((B, capacity), dtype=torch.int32, device=dev),
        "k": torch.empty((B, capacity, row), dtype=K.dtype, device=dev) if want_kv else None,
        "v": torch.empty((B, capacity, row), dtype=V.dtype, device=dev) if want_kv else None,
        "count": torch.empty(B, dtype=torch.int32, device=dev),
        "total": torch.empty(B, dtype=torch.int32, device=dev),
        }
    _check(lib().ttt_surprisal_route(
        _ptr(loss), _ptr(K), _ptr(V), _dtype_code(K), B, T, H, dh, chunk, float(pct),
        float(ema), float(ratio), capacity, _ptr(out["tau"]), _ptr(out["mask"]),
        _ptr(out["idx"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["count"]),
        _ptr(out["total"]), _stream(loss)))
    return out


def lm_target(X0, conv_w, W_target, chunk: int, *, out_dtype=None, V_hat=None, workspace=None):
    """LM-aligned target V_hat = Conv1D(X0) W_target with chunk-end padding. X0 [B,T,d_in] or
    [T,d_in] bf16; conv_w [width, d_in] fp32 (offsets +1 .. +width); W_target [d_in, d_out]
    bf16. Returns V_hat [B,T,d_out] (bf16 unless out_dtype / V_hat say otherwise)."""
    torch = _torch()
    X0 = _as3(_dev(X0, "X0"))
    _dev(conv_w, "conv_w")
    _dev(W_target, "W_target")
    if conv_w.dtype != torch.float32 or conv_w.dim() != 2:
        raise ValueError("conv_w must be float32 [width, d_in]")
    if W_target.dim() != 2:
        raise ValueError("W_target must be [d_in, d_out]")
    B, T, d_in = X0.shape
    width = conv_w.shape[0]
    d_out = W_target.shape[1]
    if conv_w.shape[1] != d_in or W_target.shape[0] != d_in:
        raise ValueError("conv_w and W_target must match X0's d_in")
    if _dtype_code(W_target) != TTT_BF16:
        raise ValueError("W_target must be bfloat16")
    if V_hat is None:
        od = out_dtype or torch.bfloat16
        V_hat = torch.empty((B, T, d_out), dtype=od, device=X0.device)
    need = lib().ttt_lm_target_workspace(B, T, d_in, d_out)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=X0.device)
    _check(lib().ttt_lm_target(
        _ptr(X0), _dtype_code(X0), _ptr(conv_w), width, _ptr(W_target), _ptr(_dev(V_hat, "V_hat")),
        _dtype_code(V_hat), B, T, d_in, d_out, chunk, _ptr(workspace), workspace.numel(),
        _stream(X0)))
    return V_hat


def gated_z(X, W_gu, *, out_dtype=None, Z=None):
    """Gated-MLP activation Z = SiLU(X W_gate) * (X W_up). X [B,T,d_model] or [T,d_model] bf16;
    W_gu [2 d_ff, d_model] bf16 in linear-layer storage: rows 0 .. d_ff-1 are W_gate^T, rows
    d_ff .. 2 d_ff-1 are W_up^T. Returns Z [B,T,d_ff] (bf16 unless out_dtype / Z say otherwise)."""
    torch = _torch()
    X = _as3(_dev(X, "X"))
    _dev(W_gu, "W_gu")
    if W_gu.dim() != 2 or W_gu.shape[0] % 2:
        raise ValueError("W_gu must be [2 d_ff, d_model]")
    if _dtype_code(W_gu) != TTT_BF16:
        raise ValueError("W_gu must be bfloat16")
    B, T, d_model = X.shape
    d_ff = W_gu.shape[0] // 2
    if W_gu.shape[1] != d_model:
        raise ValueError("W_gu rows must have X's d_model entries")
    if Z is None:
        Z = torch.empty((B, T, d_ff), dtype=out_dtype or torch.bfloat16, device=X.device)
    _check(lib().ttt_gated_z(_ptr(X), _dtype_code(X), _ptr(W_gu), _ptr(_dev(Z, "Z")),
                             _dtype_code(Z), B, T, d_model, d_ff, _stream(X)))
    return Z


def cache_readout(Q, K, V, routed_mask, ttt_out, alpha, H: int, chunk: int, capacity: int,
                  scale=None, *, out=None):
    """SR residual-cache readout: out = ttt_out + clamp(alpha, 0, 1) * softmax attention of Q
    over the cache each token's routing chunk starts with. Q, K, V [B,T,H*dh] bf16;
    routed_mask [B,T] uint8; ttt_out [B,T,H*dh] bf16 or fp32; alpha [H*dh] fp32. `out` may be
    ttt_out (in place). Returns out."""
    torch = _torch()
    Q, K, V, ttt_out = (_as3(_dev(t, n)) for t, n in
                        ((Q, "Q"), (K, "K"), (V, "V"), (ttt_out, "ttt_out")))
    _dev(routed_mask, "routed_mask")
    _dev(alpha, "alpha")
    B, T, HD = Q.shape
    if HD % H:
        raise ValueError("Q's last dimension must be H * dh")
    dh = HD // H
    for t, n in ((K, "K"), (V, "V"), (ttt_out, "ttt_out")):
        if tuple(t.shape) != (B, T, HD):
            raise ValueError(f"{n} must have Q's shape")
    if routed_mask.dtype != torch.uint8 or routed_mask.numel() != B * T:
        raise ValueError("routed_mask must be uint8 [B, T]")
    if alpha.dtype != torch.float32 or alpha.numel() != HD:
        raise ValueError("alpha must be float32 [H * dh]")
    if out is None:
        out = torch.empty_like(ttt_out)
    if scale is None:
        scale = 1.0 / dh ** 0.5
    _check(lib().ttt_cache_readout(
        _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q), _ptr(routed_mask), _ptr(ttt_out),
        _ptr(_dev(out, "out")), _dtype_code(out), _ptr(alpha), B, T, H, dh, chunk, capacity,
        float(scale), _stream(Q)))
    return out
