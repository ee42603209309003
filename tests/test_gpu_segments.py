"""The bf16 scan with a workspace below the one-pass size runs over segments of whole groups of
chunks, each resuming from the state the previous one ended with. Checked against the oracle
element by element (the same bound as one pass), and against the one-pass result, for the
state carried in W_final or in the workspace, a shared W0 with B > 1, a ragged last segment, and
the 128k-token long-context workload with a workspace of about a nineteenth of its one-pass
size."""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.inplace as oi
from helpers import TOL_BF16, assert_close, dev, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("T,C,D,F,B,shared,final,groups", [
    (5000, 512, 256, 512, 2, True, True, 2),     # shared W0, state in W_final, ragged end
    (5000, 512, 256, 512, 2, True, False, 1),    # state in the workspace, one group a segment
    (6144, 256, 320, 544, 1, False, True, 3),    # ragged tiles, three-group segments
])
def test_segmented_scan_matches_the_oracle(T, C, D, F, B, shared, final, groups):
    import torch
    print(f"case: bf16 segmented T={T} C={C} D={D} F={F} B={B} shared={shared} "
          f"W_final={final} groups/segment={groups}", flush=True)
    inp = gen.inplace_mlp(T, D, F, C, eta=2e-3, B=B, seed_base=400, shared_w0=shared)
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    full = ttt.chunk_scan_workspace_bytes(B, T, F, D, C, torch.bfloat16)
    mn = ttt.chunk_scan_workspace_bytes(B, T, F, D, C, torch.bfloat16, minimum=True)
    assert mn < full
    # a workspace that holds the operands of `groups` groups of 1024 tokens (both chunk sizes
    # group to 1024), and the fp32 state when W_final is not given
    state = 0 if final else -(-B * D * F * 4 // 256) * 256
    size = -(-ttt.chunk_scan_workspace_bytes(B, groups * 1024, F, D, C, torch.bfloat16)
             // 256) * 256 + state
    assert size < full
    ws = torch.empty(size, dtype=torch.uint8, device="cuda")
    O1, W1 = ttt.chunk_scan(Z, V, W0, C, inp.eta)                      # one pass
    O, W = ttt.chunk_scan(Z, V, W0, C, inp.eta, workspace=ws, final_state=final)
    torch.cuda.synchronize()
    Oref, Wref = oi.chunk_scan_batched(gen.bf16_bits_to_f32(inp.Z), gen.bf16_bits_to_f32(inp.V),
                                       inp.W0, C, inp.eta)
    assert_close(host_f64(O), Oref, TOL_BF16, "O (segmented) vs oracle")
    assert_close(host_f64(O), host_f64(O1), TOL_BF16, "O (segmented) vs one pass")
    if final:
        assert_close(host_f64(W), Wref, TOL_BF16, "W_final (segmented) vs oracle")
        assert_close(host_f64(W) - host_f64(W0), Wref - inp.W0, TOL_BF16, "W_final - W0")


@pytest.mark.timeout(600)
def test_long_context_in_a_bounded_workspace():
    """T=131072, C=1024, 2560/9728 (the long-context workload) with a 360 MiB workspace instead of
    the 6.8 GiB a single pass takes, against the oracle's sequential scan, every element."""
    import torch
    T, C, D, F = 131072, 1024, 2560, 9728
    full = ttt.chunk_scan_workspace_bytes(1, T, F, D, C, torch.bfloat16)
    mn = ttt.chunk_scan_workspace_bytes(1, T, F, D, C, torch.bfloat16, minimum=True)
    cap = 360 << 20
    assert mn <= cap < full / 18
    print(f"case: bf16 T={T} C={C} 2560/9728 in a {cap >> 20} MB workspace "
          f"(one pass: {full >> 20} MB)", flush=True)
    inp = gen.inplace_mlp(T, D, F, C, eta=1e-4, seed_base=30)
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    ws = torch.empty(cap, dtype=torch.uint8, device="cuda")
    O, W = ttt.chunk_scan(Z, V, W0, C, 1e-4, workspace=ws)
    torch.cuda.synchronize()
    del Z, V, ws
    o, w = host_f64(O)[0], host_f64(W)[0]
    del O, W
    print("case: full oracle scan", flush=True)
    Oref, Wref = oi.chunk_scan(gen.bf16_bits_to_f32(inp.Z[0]), gen.bf16_bits_to_f32(inp.V[0]),
                               inp.W0, C, 1e-4)
    assert_close(o, Oref, TOL_BF16, "O (every element)")
    assert_close(w, Wref, TOL_BF16, "W_final (every element)")
    assert_close(w - inp.W0, Wref - inp.W0, TOL_BF16, "W_final - W0 (every element)")
