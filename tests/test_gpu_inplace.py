"""GPU parity of ttt_chunk_scan against the fp64 oracle (called through the C ABI).

Small cases span several 256x256 tiles with ragged edges and compare every element; so do the
32k-token case at the Qwen3-4B-like MLP shape (the benchmark's workload and launch
configuration) and the 128k-token long-context case, against the oracle's sequential scan of the
whole sequence.
"""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.inplace as oi
from helpers import TOL_BF16, TOL_F32, assert_close, dev, host_bits, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _oracle(inp):
    B = inp.Z.shape[0]
    Os, Ws = [], []
    for b in range(B):
        o, w = oi.chunk_scan(inp.z_f64(b), inp.v_f64(b), inp.w0_f64(b), inp.chunk, inp.eta)
        Os.append(o)
        Ws.append(w)
    return np.stack(Os), np.stack(Ws)


def _run(inp, out_dtype=None, **kw):
    import torch
    Z, V = dev(inp.Z, inp.dtype), dev(inp.V, inp.dtype)
    W0 = dev(inp.W0, "f32")
    od = None if out_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    O, W = ttt.chunk_scan(Z, V, W0, inp.chunk, inp.eta, out_dtype=od, **kw)
    torch.cuda.synchronize()
    return O, W, W0


@pytest.fixture
def group_tokens():
    """Sets the bf16 scan's group size through the test-only override (None: the default) and
    restores the defaults afterwards."""
    def set_(n):
        ttt.scan_test_overrides(group_tokens=0 if n is None else n)
    yield set_
    ttt.scan_test_overrides()


# ---------------------------------------------------------------- fp32 path -----------------
def test_tiny_fp32_config():
    print("case: fp32 T=1024 C=64 d_model=64 d_ff=256 eta=1e-3", flush=True)
    inp = gen.inplace_f32(1024, 256, 64, 64, 1e-3)
    O, W, _ = _run(inp)
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(O), Oref, TOL_F32, "O")
    assert_close(host_f64(W), Wref, TOL_F32, "W_final")
    assert_close(host_f64(W)[0] - inp.W0, Wref[0] - inp.W0, TOL_F32, "W_final - W0")


@pytest.mark.parametrize("T,C,D,F,B,shared", [
    (1000, 64, 80, 272, 1, True),      # ragged last chunk, ragged 64-tiles
    (333, 50, 16, 48, 2, False),       # per-sequence state
    (200, 256, 32, 64, 2, True),       # chunk >= T
    (257, 1, 16, 32, 1, True),         # token-by-token
])
def test_fp32_edge_cases(T, C, D, F, B, shared):
    print(f"case: fp32 T={T} C={C} D={D} F={F} B={B} shared={shared}", flush=True)
    inp = gen.inplace_f32(T, F, D, C, 2e-3, B=B, seeds=(101, 102, 103), shared_w0=shared)
    O, W, _ = _run(inp)
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(O), Oref, TOL_F32, "O")
    assert_close(host_f64(W), Wref, TOL_F32, "W_final")


def test_fp32_eta_zero_and_inplace_state():
    inp = gen.inplace_f32(512, 64, 32, 64, 0.0, seeds=(7, 8, 9))
    O, W, W0 = _run(inp)
    np.testing.assert_array_equal(host_bits(W)[0], inp.W0)
    assert_close(host_f64(O)[0], inp.z_f64(0) @ inp.W0.astype(np.float64).T, TOL_F32, "O")
    import torch
    inp.eta = 1e-3
    Wio = W0.clone()
    O2, W2 = ttt.chunk_scan(dev(inp.Z, "f32"), dev(inp.V, "f32"), Wio, inp.chunk, inp.eta,
                            W_final=Wio)
    torch.cuda.synchronize()
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(Wio), Wref[0], TOL_F32, "in-place W_final")
    assert_close(host_f64(O2), Oref, TOL_F32, "O")


# ---------------------------------------------------------------- bf16 path -----------------
@pytest.mark.parametrize("T,C,D,F,group", [
    (2048, 512, 256, 512, None),       # default grouping (2 chunks per group)
    (2048, 512, 272, 528, 512),        # one chunk per group, ragged 256-tiles
    (1536, 256, 256, 512, 768),        # three chunks per group
    (1000, 100, 64, 96, 300),          # chunk not a multiple of 8, ragged T, small tiles
    (700, 128, 48, 160, 100000),       # a single group holding every chunk
    (4000, 512, 272, 576, None),       # 4 groups, the state chain split after group 2, ragged
    (8192, 512, 256, 512, 2048),       # 4 groups of 32 steps each
    (2048, 16, 256, 512, None),        # 64 chunks per group: per-element correction mask,
                                       # four-wave apply (chunk not a whole 32-token step)
    (3072, 64, 320, 512, None),        # 16 chunks per group, eight-wave apply, ragged d_model
    (2000, 512, 256, 512, None),       # T not a whole 32-token step: the state chain's last step
                                       # holds 16 valid tokens (the staged V_hat^T is zero past T)
])
def test_bf16_parity(T, C, D, F, group, group_tokens):
    print(f"case: bf16 T={T} C={C} D={D} F={F} group_tokens={group}", flush=True)
    group_tokens(group)
    inp = gen.inplace_mlp(T, D, F, C, eta=3e-3, seed_base=300)
    O, W, _ = _run(inp)
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(O), Oref, TOL_BF16, "O")
    assert_close(host_f64(W), Wref, TOL_BF16, "W_final")
    assert_close(host_f64(W)[0] - inp.W0, Wref[0] - inp.W0, TOL_BF16, "W_final - W0")


def test_bf16_batch_shared_state_fp32_output():
    inp = gen.inplace_mlp(1024, 128, 256, 256, eta=3e-3, B=2, seed_base=310)
    O, W, _ = _run(inp, out_dtype="f32")
    Oref, Wref = _oracle(inp)
    assert O.dtype.is_floating_point and O.element_size() == 4
    assert_close(host_f64(O), Oref, TOL_BF16, "O")
    assert_close(host_f64(W), Wref, TOL_BF16, "W_final")


def test_bf16_per_sequence_state_several_groups():
    # B = 2 with its own W0 per sequence on the unmasked path: each sequence's first state-chain
    # workgroups write that sequence's group-0 snapshot
    print("case: bf16 B=2 T=2048 C=256 D=256 F=512 per-sequence W0", flush=True)
    inp = gen.inplace_mlp(2048, 256, 512, 256, eta=3e-3, B=2, seed_base=312, shared_w0=False)
    O, W, _ = _run(inp)
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(O), Oref, TOL_BF16, "O")
    assert_close(host_f64(W), Wref, TOL_BF16, "W_final")


@pytest.mark.parametrize("T", [2048, 512])
def test_bf16_without_final_state_is_bitwise_the_same_output(T):
    # no W_final: with several groups the state chain still runs (for the snapshots); with one
    # group it does not run at all and the apply takes bf16(W0) from the separate conversion
    print(f"case: bf16 T={T} C=256 D=256 F=512 final_state=False", flush=True)
    inp = gen.inplace_mlp(T, 256, 512, 256, eta=3e-3, seed_base=314)
    O1, W1, _ = _run(inp)
    O2, W2, _ = _run(inp, final_state=False)
    assert W2 is None
    np.testing.assert_array_equal(host_bits(O2), host_bits(O1))
    Oref, _ = _oracle(inp)
    assert_close(host_f64(O2), Oref, TOL_BF16, "O")


def test_bf16_eta_zero_keeps_state_bits():
    inp = gen.inplace_mlp(1024, 128, 256, 256, eta=0.0, seed_base=320)
    O, W, _ = _run(inp)
    np.testing.assert_array_equal(host_bits(W)[0], inp.W0)
    assert_close(host_f64(O)[0], inp.z_f64(0) @ inp.W0.astype(np.float64).T, TOL_BF16, "O")


def test_bf16_eta_zero_copies_shared_state():
    # eta = 0, batch 2 sharing W0, W_final a separate buffer, several groups
    import torch
    inp = gen.inplace_mlp(3072, 128, 256, 512, eta=0.0, B=2, seed_base=321)
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    Wf = torch.full((2, 128, 256), float("nan"), dtype=torch.float32, device=Z.device)
    O, W = ttt.chunk_scan(Z, V, W0, 512, 0.0, W_final=Wf)
    torch.cuda.synchronize()
    for b in range(2):
        np.testing.assert_array_equal(host_bits(W)[b], inp.W0)
        assert_close(host_f64(O)[b], inp.z_f64(b) @ inp.W0.astype(np.float64).T, TOL_BF16, "O")


def test_bf16_negative_eta():
    inp = gen.inplace_mlp(4096, 128, 256, 512, eta=-2e-3, seed_base=325)
    O, W, _ = _run(inp)
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(O), Oref, TOL_BF16, "O")
    assert_close(host_f64(W)[0] - inp.W0, Wref[0] - inp.W0, TOL_BF16, "W_final - W0")


@pytest.mark.parametrize("group", [None, 256])
def test_bf16_causality(group, group_tokens):
    # Changing V_hat inside chunk i leaves every output row of chunks <= i bit-identical.
    group_tokens(group)
    import torch
    inp = gen.inplace_mlp(2048, 128, 256, 256, eta=3e-3, seed_base=330)
    O1, _, _ = _run(inp)
    C = inp.chunk
    for i in (1, 4):
        V2 = inp.V.copy()
        V2[0, i * C:(i + 1) * C] ^= np.uint16(0x0040)        # flip a mantissa bit
        Z, W0 = dev(inp.Z, "bf16"), dev(inp.W0, "f32")
        O2, _ = ttt.chunk_scan(Z, dev(V2, "bf16"), W0, C, inp.eta)
        torch.cuda.synchronize()
        a, b = host_bits(O1)[0], host_bits(O2)[0]
        np.testing.assert_array_equal(a[:(i + 1) * C], b[:(i + 1) * C])
        assert (a[(i + 1) * C:(i + 2) * C] != b[(i + 1) * C:(i + 2) * C]).any()


def test_bf16_resume_and_chunk_size_invariance():
    import torch
    inp = gen.inplace_mlp(2048, 128, 256, 512, eta=3e-3, seed_base=340)
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    O, W = ttt.chunk_scan(Z, V, W0, 512, inp.eta)
    Oa, Wa = ttt.chunk_scan(Z[:, :1024].contiguous(), V[:, :1024].contiguous(), W0, 512, inp.eta)
    Ob, Wb = ttt.chunk_scan(Z[:, 1024:].contiguous(), V[:, 1024:].contiguous(), Wa[0].contiguous(),
                            512, inp.eta)
    _, W256 = ttt.chunk_scan(Z, V, W0, 256, inp.eta)
    torch.cuda.synchronize()
    Oref, Wref = _oracle(inp)
    assert_close(np.concatenate([host_f64(Oa), host_f64(Ob)], 1), Oref, TOL_BF16, "resumed O")
    assert_close(host_f64(Wb), Wref, TOL_BF16, "resumed W")
    assert_close(host_f64(W256), Wref, TOL_BF16, "W_final at C=256")


@pytest.fixture
def overrides():
    yield ttt.scan_test_overrides
    ttt.scan_test_overrides()


def test_bf16_token_split_is_bitwise_the_unsplit_chain(overrides):
    """The state chain's token split (first half hands its fp32 state to the second half) gives
    the same bits as one pass over all tokens: per-sequence W0, B = 2, ragged tiles, 4 groups."""
    import torch
    print("case: bf16 B=2 T=4000 C=512 D=272 F=576 split vs unsplit", flush=True)
    inp = gen.inplace_mlp(4000, 272, 576, 512, eta=2e-3, B=2, seed_base=350, shared_w0=False)
    overrides()
    O1, W1, _ = _run(inp)
    overrides(token_split=0)
    O0, W0b, _ = _run(inp)
    overrides()
    assert np.array_equal(host_bits(O1), host_bits(O0)), "O differs between split and unsplit"
    assert torch.equal(W1, W0b), "W_final differs between split and unsplit"
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(O1), Oref, TOL_BF16, "O")
    assert_close(host_f64(W1), Wref, TOL_BF16, "W_final")


@pytest.mark.parametrize("B,shared", [(1, True), (2, False)])
def test_bf16_split_wait_bound_recomputes_the_same_bits(overrides, B, shared):
    """With the second halves' bounded wait forced to zero polls from the host, every second
    half gives up on the hand-over at once and recomputes its first half's tokens from W0: the
    outputs are the same bits as with the hand-over, and the workspace counts one event per
    second half (state tiles x sequences)."""
    import torch
    T, C, D, F = 4096, 512, 256, 512
    print(f"case: bf16 T={T} C={C} D={D} F={F} B={B}, second-half wait limit 0", flush=True)
    inp = gen.inplace_mlp(T, D, F, C, eta=2e-3, B=B, seed_base=360, shared_w0=shared)
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    ws = torch.empty(ttt.chunk_scan_workspace_bytes(B, T, F, D, C, torch.bfloat16),
                     dtype=torch.uint8, device="cuda")
    overrides()
    O_ok, W_ok = ttt.chunk_scan(Z, V, W0, C, inp.eta, workspace=ws)
    n_ok = ttt.chunk_scan_handover_timeouts(ws, B, T, F, D, C, torch.bfloat16)
    torch.cuda.synchronize()
    overrides(spin_limit=0)
    O_re, W_re = ttt.chunk_scan(Z, V, W0, C, inp.eta, workspace=ws)
    n_re = ttt.chunk_scan_handover_timeouts(ws, B, T, F, D, C, torch.bfloat16)
    torch.cuda.synchronize()
    overrides()
    assert int(n_ok.item()) == 0
    assert int(n_re.item()) == B * (F // 256) * (D // 256), int(n_re.item())
    assert np.array_equal(host_bits(O_re), host_bits(O_ok)), "O differs after recomputation"
    assert torch.equal(W_re, W_ok), "W_final differs after recomputation"
    Oref, Wref = _oracle(inp)
    assert_close(host_f64(O_re), Oref, TOL_BF16, "O")
    assert_close(host_f64(W_re), Wref, TOL_BF16, "W_final")


def _full_workload_check(T, C, seed_base, split):
    """Every element of O, W_final and W_final - W0 at a benchmark shape (d_model = 2560,
    d_ff = 9728, eta = 1e-4) against the oracle's sequential scan over the whole sequence, plus
    a look at the rows on both sides of the state chain's token split."""
    import torch
    print(f"case: bf16 T={T} C={C} D=2560 F=9728 (generating inputs)", flush=True)
    inp = gen.inplace_mlp(T, 2560, 9728, C, eta=1e-4, seed_base=seed_base)
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    O, W = ttt.chunk_scan(Z, V, W0, C, 1e-4)
    torch.cuda.synchronize()
    del Z, V
    o, w = host_f64(O)[0], host_f64(W)[0]
    del O, W
    print("case: full oracle scan", flush=True)
    z = gen.bf16_bits_to_f32(inp.Z[0])
    v = gen.bf16_bits_to_f32(inp.V[0])
    Oref, Wref = oi.chunk_scan(z, v, inp.W0, C, 1e-4)
    del z, v
    assert_close(o, Oref, TOL_BF16, "O (every element)")
    assert_close(o[split - C:split + C], Oref[split - C:split + C], TOL_BF16,
                 f"O, the chunks on both sides of token {split}")
    assert_close(w, Wref, TOL_BF16, "W_final (every element)")
    assert_close(w - inp.W0, Wref - inp.W0, TOL_BF16, "W_final - W0 (every element)")


@pytest.mark.timeout(300)
def test_bench_workload_full():
    """T=32768, C=512 (64 chunks), the benchmark's workload and launch configuration: 32 groups
    of 1024 tokens, token split of the state chain at 16384."""
    _full_workload_check(32768, 512, 20, 16384)


@pytest.mark.timeout(600)
def test_long_context_workload_full():
    """T=131072, C=1024 (128 chunks), the same gated-MLP and target generators with seeds
    31..37: one chunk per group, token split at 65536."""
    _full_workload_check(131072, 1024, 30, 65536)
