"""Helpers shared by the GPU tests: moving generator output to the device and the error metric.

Agreement metric (the tolerance reading used throughout): the normwise max relative error
max|y - y_ref| / max|y_ref| over a tensor; bf16-input paths must stay within 2e-2, the fp32
path within 1e-4, and integer outputs must match exactly.
"""
import numpy as np
import pytest

TOL_BF16 = 2e-2
TOL_F32 = 1e-4


def have_gpu() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


requires_gpu = pytest.mark.skipif(not have_gpu(), reason="no GPU visible")


def dev(a, dtype: str):
    """numpy array (uint16 bf16 bits or float32) -> torch tensor on cuda:0."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to("cuda:0")


def host_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def host_bits(t) -> np.ndarray:
    import torch
    t = t.detach().to("cpu")
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def rel_err(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(y - ref).max() / (den if den > 0 else 1.0))


def assert_close(y, ref, tol, what=""):
    e = rel_err(y, ref)
    print(f"  {what}: normwise max rel err = {e:.3e} (tol {tol:.0e})", flush=True)
    assert np.all(np.isfinite(y)), f"{what}: non-finite values"
    assert e <= tol, f"{what}: {e:.3e} > {tol:.0e}"
