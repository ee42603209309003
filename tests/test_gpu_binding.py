"""The Python binding refuses, before any launch, tensors whose dtype, shape or device the C ABI
cannot check (it receives only pointers): each case would otherwise read or write past a
buffer."""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
from helpers import requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _scan_inputs(B=2, T=512, F=256, D=128):
    import torch
    g = torch.Generator(device="cpu").manual_seed(5)
    Z = torch.randn(B, T, F, generator=g).to(torch.bfloat16).cuda()
    V = torch.randn(B, T, D, generator=g).to(torch.bfloat16).cuda()
    W0 = (0.02 * torch.randn(D, F, generator=g)).cuda()
    return Z, V, W0


@pytest.mark.parametrize("case", ["vhat_dtype", "w0_batch_1", "w0_batch_3", "o_shape", "o_dtype",
                                  "wf_dtype", "wf_shape", "w0_cpu"])
def test_scan_binding_rejects_mismatched_tensors(case):
    import torch
    Z, V, W0 = _scan_inputs()
    B, T, F = Z.shape
    D = V.shape[2]
    kw = {}
    if case == "vhat_dtype":
        V = V.float()
    elif case == "w0_batch_1":
        W0 = W0.unsqueeze(0).contiguous()                    # [1, D, F] with B = 2
    elif case == "w0_batch_3":
        W0 = W0.expand(3, D, F).contiguous()
    elif case == "o_shape":
        kw["O"] = torch.empty(B, T - 1, D, dtype=torch.bfloat16, device="cuda")
    elif case == "o_dtype":
        kw["O"] = torch.empty(B, T, D, dtype=torch.float16, device="cuda")
    elif case == "wf_dtype":
        kw["W_final"] = torch.empty(B, D, F, dtype=torch.bfloat16, device="cuda")
    elif case == "wf_shape":
        kw["W_final"] = torch.empty(1, D, F, dtype=torch.float32, device="cuda")
    elif case == "w0_cpu":
        W0 = W0.cpu()
    with pytest.raises((ValueError, TypeError)):
        ttt.chunk_scan(Z, V, W0, 64, 1e-3, **kw)


@pytest.mark.parametrize("case", ["o_shape", "o_dtype", "wf_shape", "loss_shape", "loss_dtype"])
def test_linear_binding_rejects_mismatched_outputs(case):
    import torch
    B, T, H, dh = 1, 64, 2, 64
    Q = torch.randn(B, T, H, dh).to(torch.bfloat16).cuda()
    kw = {}
    if case == "o_shape":
        kw["O"] = torch.empty(B, T, H, 32, dtype=torch.bfloat16, device="cuda")
    elif case == "o_dtype":
        kw["O"] = torch.empty(B, T, H, dh, dtype=torch.float16, device="cuda")
    elif case == "wf_shape":
        kw["W_final"] = torch.empty(B, H, dh, dh - 1, dtype=torch.float32, device="cuda")
    elif case == "loss_shape":
        kw["loss"] = torch.empty(B, T, H + 1, dtype=torch.float32, device="cuda")
    elif case == "loss_dtype":
        kw["loss"] = torch.empty(B, T, H, dtype=torch.bfloat16, device="cuda")
    with pytest.raises((ValueError, TypeError)):
        ttt.linear_minibatch(Q, Q, Q, 16, 0.1, **kw)


@pytest.mark.parametrize("case", ["idx_dtype", "k_dtype", "tau_shape", "mask_dtype", "kv_shape"])
def test_route_binding_rejects_mismatched_outputs(case):
    import torch
    B, T, H, dh, cap = 1, 256, 2, 64, 8
    loss = torch.rand(B, T, H, device="cuda")
    K = torch.randn(B, T, H * dh).to(torch.bfloat16).cuda()
    V = K.clone()
    out = ttt.surprisal_route(loss, K, V, 64, capacity=cap)
    if case == "idx_dtype":
        out["idx"] = out["idx"].to(torch.int64)
    elif case == "k_dtype":
        out["k"] = out["k"].float()
    elif case == "tau_shape":
        out["tau"] = torch.empty(B, T // 64 + 1, device="cuda")
    elif case == "mask_dtype":
        out["mask"] = out["mask"].to(torch.int32)
    elif case == "kv_shape":
        V = V[:, :128].contiguous()
    with pytest.raises((ValueError, TypeError)):
        ttt.surprisal_route(loss, K, V, 64, capacity=cap, out=out)
