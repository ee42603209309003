"""HIP graph capture of the entry points, as a serving loop would use them: each call is captured
once into a torch CUDA graph (on torch's capture stream, with every buffer allocated before the
capture) and the graph is replayed several times. Between the replays the program does its own
eager work: library calls on other inputs that reuse the same workspace or static scratch, torch
kernels and host synchronisation. Every replay must equal the eager result bit for bit (the same
kernels on the same inputs), and a replay after an input buffer was overwritten in place must equal
the eager result on the new contents. The library clears what must start at zero (the scan's
hand-over flags, the routing outputs' empty slots) with its own kernels, not with memset nodes.
"""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
from helpers import dev, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

REPLAYS = 4


def _same(a, b) -> bool:
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    return torch.equal(a, b)


def _eager_noise():
    import torch
    x = torch.randn(1 << 20, device="cuda")
    y = (x * 2 + 1).sum()
    torch.cuda.synchronize()
    return float(y)


def _scan_inputs(seed, T=4096, C=512, D=512, F=1024):
    inp = gen.inplace_mlp(T, D, F, C, eta=2e-3, seed_base=seed)
    return inp, dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")


def test_scan_graph_replays():
    import torch
    # 4 groups of 1024 tokens: correction blocks and the update's token split (hand-over flags)
    print("case: graph ttt_chunk_scan bf16 T=4096 C=512 D=512 F=1024", flush=True)
    T, C, D, F = 4096, 512, 512, 1024
    inp, Z, V, W0 = _scan_inputs(700)
    _, Z2, V2, _ = _scan_inputs(710)
    need = ttt.lib().ttt_chunk_scan_workspace(1, T, F, D, C, 1)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    O_ref, W_ref = ttt.chunk_scan(Z, V, W0, C, inp.eta, workspace=ws)
    O2_ref, W2_ref = ttt.chunk_scan(Z2, V, W0, C, inp.eta, workspace=ws)
    O = torch.empty_like(O_ref)
    Wf = torch.empty_like(W_ref)
    O_e = torch.empty_like(O_ref)
    W_e = torch.empty_like(W_ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ttt.chunk_scan(Z, V, W0, C, inp.eta, O=O, W_final=Wf, workspace=ws)
    for r in range(REPLAYS):
        O.fill_(float("nan"))
        Wf.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert _same(O, O_ref) and _same(Wf, W_ref), f"replay {r} differs from the eager call"
        # eager work between replays: another scan through the same workspace, torch kernels
        ttt.chunk_scan(Z2, V2, W0, C, inp.eta, O=O_e, W_final=W_e, workspace=ws)
        _eager_noise()
    Z.copy_(Z2)  # the graph reads the live input buffer
    g.replay()
    torch.cuda.synchronize()
    assert _same(O, O2_ref) and _same(Wf, W2_ref), "replay on new input contents differs"


def test_scan_noalloc_graph_replays():
    import torch
    print("case: graph ttt_chunk_scan_noalloc bf16 T=4096 C=512 D=512 F=1024", flush=True)
    inp, Z, V, W0 = _scan_inputs(720)
    _, Z2, V2, _ = _scan_inputs(730)
    C = 512
    O_ref, W_ref = ttt.chunk_scan(Z, V, W0, C, inp.eta)
    O = torch.empty_like(O_ref)
    Wf = torch.empty_like(W_ref)
    O_e = torch.empty_like(O_ref)
    W_e = torch.empty_like(W_ref)
    # first call outside the capture (the library finds the scratch's device address once)
    ttt.chunk_scan_noalloc(Z, V, W0, C, inp.eta, O=O, W_final=Wf)
    torch.cuda.synchronize()
    assert _same(O, O_ref) and _same(Wf, W_ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ttt.chunk_scan_noalloc(Z, V, W0, C, inp.eta, O=O, W_final=Wf)
    for r in range(REPLAYS):
        O.fill_(float("nan"))
        Wf.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert _same(O, O_ref) and _same(Wf, W_ref), f"replay {r} differs from the eager call"
        # the same static scratch used by an eager call in between (stream-ordered, no overlap)
        ttt.chunk_scan_noalloc(Z2, V2, W0, C, inp.eta, O=O_e, W_final=W_e)
        _eager_noise()


def test_linear_and_route_graph_replays():
    import torch
    print("case: graph ttt_linear_minibatch b=16 + ttt_surprisal_route chunk 64, B=2 T=1024 4x64",
          flush=True)
    inp = gen.route_inputs(B=2, T=1024, d_model=256, H=4, dh=64, seed_base=740)
    Q, K, V = dev(inp.Q, "bf16"), dev(inp.K, "bf16"), dev(inp.V, "bf16")
    inp2 = gen.route_inputs(B=2, T=1024, d_model=256, H=4, dh=64, seed_base=750)
    Q2, K2, V2 = dev(inp2.Q, "bf16"), dev(inp2.K, "bf16"), dev(inp2.V, "bf16")
    O_ref, W_ref, L_ref = ttt.linear_minibatch(Q, K, V, 16, 0.01)
    r_ref = ttt.surprisal_route(L_ref, K, V, 64)
    O = torch.empty_like(O_ref)
    Wf = torch.empty_like(W_ref)
    L = torch.empty_like(L_ref)
    r_out = ttt.surprisal_route(L_ref, K, V, 64)  # allocates the output tensors reused below
    torch.cuda.synchronize()
    assert r_ref["count"].sum().item() > 0, "no token routed: the case checks nothing"
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ttt.linear_minibatch(Q, K, V, 16, 0.01, O=O, W_final=Wf, loss=L)
        ttt.surprisal_route(L, K, V, 64, out=r_out)
    for r in range(REPLAYS):
        O.fill_(float("nan"))
        L.fill_(float("nan"))
        for t in r_out.values():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert _same(O, O_ref) and _same(Wf, W_ref) and _same(L, L_ref), f"TTT-Linear replay {r}"
        for k, t in r_ref.items():
            assert _same(r_out[k], t), f"routing output {k} differs in replay {r}"
        # eager work in between: the same entry points on other inputs
        _, _, L2 = ttt.linear_minibatch(Q2, K2, V2, 16, 0.01)
        ttt.surprisal_route(L2, K2, V2, 64)
        _eager_noise()
    # the graph reads the live buffers: new contents of Q, K, V
    Q.copy_(Q2)
    K.copy_(K2)
    V.copy_(V2)
    O2_ref, W2_ref, L2_ref = ttt.linear_minibatch(Q2, K2, V2, 16, 0.01)
    r2_ref = ttt.surprisal_route(L2_ref, K2, V2, 64)
    g.replay()
    torch.cuda.synchronize()
    assert _same(O, O2_ref) and _same(Wf, W2_ref) and _same(L, L2_ref)
    for k, t in r2_ref.items():
        assert _same(r_out[k], t), f"routing output {k} differs on new input contents"
