"""ttt_chunk_scan_noalloc (the scan with its workspace in the library's static device scratch,
for callers that cannot allocate) against ttt_chunk_scan with a caller workspace, through the C
ABI: two calls in a row, the second on a smaller input, each bit for bit equal to the existing
entry point's result (the same kernels on the same inputs) and within the bf16 bound of the
oracle. (The refusal of shapes whose workspace exceeds the scratch is a host check, tested
without a GPU in test_abi.py.)"""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.inplace as oi
from helpers import TOL_BF16, assert_close, dev, host_bits, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _case(T, C, D, F, B, seed, shared=True):
    import torch
    inp = gen.inplace_mlp(T, D, F, C, eta=2e-3, B=B, seed_base=seed, shared_w0=shared)
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    need = ttt.chunk_scan_workspace_bytes(B, T, F, D, C, torch.bfloat16)
    assert 0 < need <= ttt.lib().ttt_chunk_scan_workspace(B, T, F, D, C, 1)
    O_ref, W_ref = ttt.chunk_scan(Z, V, W0, C, inp.eta)
    O = torch.full((B, T, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    Wf = torch.full((B, D, F), float("nan"), dtype=torch.float32, device="cuda")
    ttt.chunk_scan_noalloc(Z, V, W0, C, inp.eta, O=O, W_final=Wf)
    torch.cuda.synchronize()
    return inp, O, Wf, O_ref, W_ref


def test_noalloc_matches_the_workspace_entry_point_twice():
    import torch
    # first call: 4 groups (token split, correction blocks), per-sequence W0, B = 2
    print("case: noalloc bf16 B=2 T=4096 C=512 D=256 F=512", flush=True)
    inp, O, Wf, O_ref, W_ref = _case(4096, 512, 256, 512, 2, 380, shared=False)
    assert np.array_equal(host_bits(O), host_bits(O_ref)), "O differs from ttt_chunk_scan"
    assert torch.equal(Wf, W_ref), "W_final differs from ttt_chunk_scan"
    Oo, Wo = oi.chunk_scan_batched(gen.bf16_bits_to_f32(inp.Z), gen.bf16_bits_to_f32(inp.V),
                                   inp.W0, 512, inp.eta)
    assert_close(host_f64(O), Oo, TOL_BF16, "O vs oracle")
    assert_close(host_f64(Wf), Wo, TOL_BF16, "W_final vs oracle")
    # second call, smaller input (the scratch still holds the first call's contents)
    print("case: noalloc bf16 B=1 T=1000 C=100 D=64 F=96", flush=True)
    inp, O, Wf, O_ref, W_ref = _case(1000, 100, 64, 96, 1, 390)
    assert np.array_equal(host_bits(O), host_bits(O_ref)), "O differs from ttt_chunk_scan"
    assert torch.equal(Wf, W_ref), "W_final differs from ttt_chunk_scan"
    Oo, Wo = oi.chunk_scan(inp.z_f64(0), inp.v_f64(0), inp.w0_f64(0), 100, inp.eta)
    assert_close(host_f64(O)[0], Oo, TOL_BF16, "O vs oracle")
    assert_close(host_f64(Wf)[0], Wo, TOL_BF16, "W_final vs oracle")
