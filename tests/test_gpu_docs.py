"""GPU parity of ttt_chunk_scan_docs (document-boundary reset and per-chunk update clipping)
against the fp64 oracle: both input paths, shared and per-sequence state, in-place state, the
no-op cases bit for bit against ttt_chunk_scan, documents bit for bit against separate scans,
and the 32k-token workload on sampled rows."""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.docs as od
import oracle.inplace as oi
from helpers import TOL_BF16, TOL_F32, assert_close, dev, host_bits, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(B, T, F, D, seed, dtype="bf16", shared=True):
    rng = np.random.default_rng(seed)
    Z = rng.standard_normal((B, T, F)).astype(np.float32)
    V = rng.standard_normal((B, T, D)).astype(np.float32)
    W0 = (rng.standard_normal((D, F) if shared else (B, D, F)) / np.sqrt(F)).astype(np.float32)
    if dtype == "bf16":
        Z, V = gen.f32_to_bf16_bits(Z), gen.f32_to_bf16_bits(V)
    return Z, V, W0


def _f(a):
    return gen.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def _oracle(Z, V, W0, C, eta, docs, tau):
    Os, Ws = [], []
    for b in range(Z.shape[0]):
        w0 = W0 if W0.ndim == 2 else W0[b]
        o, w = od.chunk_scan_docs(_f(Z[b]), _f(V[b]), w0, C, eta, docs[b] if docs else (), tau)
        Os.append(o)
        Ws.append(w)
    return np.stack(Os), np.stack(Ws)


def _run(Z, V, W0, C, eta, docs, tau, dtype="bf16", out_dtype=None, inplace=False):
    import torch
    Zd, Vd, W0d = dev(Z, dtype), dev(V, dtype), dev(W0, "f32")
    od_ = None if out_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    O, W = ttt.chunk_scan_docs(Zd, Vd, W0d, C, eta, doc_starts=docs, clip_tau=tau,
                               out_dtype=od_, W_final=W0d if inplace else None)
    torch.cuda.synchronize()
    return O, W


def _check(O, W, ref, W0, tol, what):
    assert_close(host_f64(O), ref[0], tol, f"{what} O")
    assert_close(host_f64(W), ref[1], tol, f"{what} W_final")
    w0 = W0 if W0.ndim == 3 else W0[None]
    assert_close(host_f64(W) - w0, ref[1] - w0, tol, f"{what} W_final - W0")


def _median_tau(Z, V, C, eta):
    n = np.concatenate([od.delta_norms(_f(Z[b]), _f(V[b]), C, eta) for b in range(Z.shape[0])])
    return float(np.median(n))


def test_documents_bf16():
    print("case: docs bf16 B=2 T=1000 F=128 D=64 C=64", flush=True)
    Z, V, W0 = _inputs(2, 1000, 128, 64, 1000)
    docs = [[256, 640], [128]]
    O, W = _run(Z, V, W0, 64, 0.02, docs, 0.0)
    _check(O, W, _oracle(Z, V, W0, 64, 0.02, docs, None), W0, TOL_BF16, "docs")


def test_clipping_bf16_half_the_chunks():
    print("case: clip bf16 B=1 T=768 F=256 D=128 C=128", flush=True)
    Z, V, W0 = _inputs(1, 768, 256, 128, 1010)
    tau = _median_tau(Z, V, 128, 0.05)
    O, W = _run(Z, V, W0, 128, 0.05, None, tau)
    ref = _oracle(Z, V, W0, 128, 0.05, None, tau)
    _check(O, W, ref, W0, TOL_BF16, "clip")
    plain = _oracle(Z, V, W0, 128, 0.05, None, None)
    got = host_f64(W)[0] - W0
    to_ref = np.abs(got - (ref[1][0] - W0)).max()
    to_plain = np.abs(got - (plain[1][0] - W0)).max()
    assert to_plain > 2 * to_ref, (to_ref, to_plain)


def test_clipping_bf16_chunk_over_two_gram_tiles_ragged():
    # C = 384: each chunk's Gram matrix spans a full and a partial 256-row block, so the norm
    # sums two diagonal tiles and one doubled off-diagonal tile; the last chunk is ragged
    print("case: clip bf16 B=1 T=1000 F=256 D=128 C=384", flush=True)
    Z, V, W0 = _inputs(1, 1000, 256, 128, 1012)
    tau = _median_tau(Z, V, 384, 0.05)
    O, W = _run(Z, V, W0, 384, 0.05, None, tau)
    _check(O, W, _oracle(Z, V, W0, 384, 0.05, None, tau), W0, TOL_BF16, "clip C=384")


def test_clipping_bf16_register_engine_norm():
    # d_ff a multiple of 16 but not of 32: the norm runs on the register-staged engine
    print("case: clip bf16 B=2 T=512 F=208 D=96 C=128", flush=True)
    Z, V, W0 = _inputs(2, 512, 208, 96, 1013)
    tau = _median_tau(Z, V, 128, 0.05)
    O, W = _run(Z, V, W0, 128, 0.05, None, tau)
    _check(O, W, _oracle(Z, V, W0, 128, 0.05, None, tau), W0, TOL_BF16, "clip F=208")


def test_strong_clipping_bf16():
    # every chunk clipped to a fifth of the smallest delta norm
    Z, V, W0 = _inputs(1, 512, 128, 64, 1015)
    n = od.delta_norms(_f(Z[0]), _f(V[0]), 64, 0.05)
    tau = 0.2 * float(n.min())
    O, W = _run(Z, V, W0, 64, 0.05, None, tau)
    ref = _oracle(Z, V, W0, 64, 0.05, None, tau)
    _check(O, W, ref, W0, TOL_BF16, "strong clip")
    d = host_f64(W)[0] - W0
    assert np.linalg.norm(d) <= 8 * tau * 1.02   # eight deltas of norm tau


def test_documents_and_clipping_per_sequence_state_fp32_output():
    print("case: docs+clip bf16 B=2 T=640 F=192 D=96 C=64 per-sequence W0", flush=True)
    Z, V, W0 = _inputs(2, 640, 192, 96, 1020, shared=False)
    docs = [[384], []]
    tau = _median_tau(Z, V, 64, 0.03)
    O, W = _run(Z, V, W0, 64, 0.03, docs, tau, out_dtype="f32")
    assert O.element_size() == 4
    _check(O, W, _oracle(Z, V, W0, 64, 0.03, docs, tau), W0, TOL_BF16, "docs+clip")


def test_fp32_path_documents_and_clipping():
    print("case: docs+clip fp32 B=2 T=200 F=32 D=16 C=16", flush=True)
    Z, V, W0 = _inputs(2, 200, 32, 16, 1030, dtype="f32")
    docs = [[64, 160], [16]]
    tau = _median_tau(Z, V, 16, 0.05)
    O, W = _run(Z, V, W0, 16, 0.05, docs, tau, dtype="f32")
    _check(O, W, _oracle(Z, V, W0, 16, 0.05, docs, tau), W0, TOL_F32, "fp32 docs+clip")


def test_in_place_state_with_documents():
    Z, V, W0 = _inputs(1, 512, 128, 64, 1040)
    docs = [[192]]
    ref = _oracle(Z, V, W0, 64, 0.02, docs, None)
    O, W = _run(Z, V, W0, 64, 0.02, docs, 0.0, inplace=True)
    assert_close(host_f64(W), ref[1], TOL_BF16, "in-place W_final")
    assert_close(host_f64(O), ref[0], TOL_BF16, "in-place O")


def test_no_documents_no_clip_is_bitwise_the_plain_scan():
    import torch
    Z, V, W0 = _inputs(2, 700, 128, 64, 1050)
    O1, W1 = _run(Z, V, W0, 64, 0.02, None, 0.0)
    O2, W2 = ttt.chunk_scan(dev(Z, "bf16"), dev(V, "bf16"), dev(W0, "f32"), 64, 0.02)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(O1), host_bits(O2))
    np.testing.assert_array_equal(host_bits(W1), host_bits(W2))
    O3, W3 = _run(Z, V, W0, 64, 0.02, [[], []], float("inf"))
    np.testing.assert_array_equal(host_bits(O3), host_bits(O2))


def test_documents_are_bitwise_separate_scans():
    import torch
    Z, V, W0 = _inputs(1, 896, 128, 64, 1060)
    O, W = _run(Z, V, W0, 64, 0.02, [[320]], 0.0)
    Oa, _ = ttt.chunk_scan(dev(Z[:, :320], "bf16"), dev(V[:, :320], "bf16"), dev(W0, "f32"), 64,
                           0.02)
    Ob, Wb = ttt.chunk_scan(dev(Z[:, 320:], "bf16"), dev(V[:, 320:], "bf16"), dev(W0, "f32"), 64,
                            0.02)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host_bits(O)[:, :320], host_bits(Oa))
    np.testing.assert_array_equal(host_bits(O)[:, 320:], host_bits(Ob))
    np.testing.assert_array_equal(host_bits(W), host_bits(Wb))


def test_documents_on_group_boundaries_are_bitwise_separate_scans():
    """Document starts on multiples of the scan's 1024-token groups run as one batched scan whose
    state chain goes back to W0 at each start; the bits equal separate scans of the documents.
    B = 2, per-sequence W0, one start exactly at the state chain's token split (2048)."""
    import torch
    print("case: docs on group boundaries bf16 B=2 T=4096 F=512 D=256 C=512", flush=True)
    Z, V, W0 = _inputs(2, 4096, 512, 256, 1070, shared=False)
    docs = [[1024, 2048], [3072]]
    O, W = _run(Z, V, W0, 512, 0.01, docs, 0.0)
    for b in range(2):
        bounds = [0] + docs[b] + [4096]
        for s, e in zip(bounds[:-1], bounds[1:]):
            Os, Ws = ttt.chunk_scan(dev(Z[b:b + 1, s:e], "bf16"), dev(V[b:b + 1, s:e], "bf16"),
                                    dev(W0[b], "f32"), 512, 0.01)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(host_bits(O)[b, s:e], host_bits(Os)[0])
        np.testing.assert_array_equal(host_bits(W)[b], host_bits(Ws)[0])
    _check(O, W, _oracle(Z, V, W0, 512, 0.01, docs, None), W0, TOL_BF16, "docs on groups")


def test_documents_inside_groups_batched():
    """Starts inside a 1024-token group on a 256-token tile edge also run as one batched scan:
    the state chain goes back to W0 before the start's first step and the tiles from the start
    on apply bf16(W0) with the correction taken from the start only. Against the oracle, plus
    the first document bit for bit against a separate scan of it (its groups fall the same way).
    B = 2, per-sequence W0; starts at offsets 256 and 512 inside groups, one on a group
    boundary at the state chain's token split (2048), and two in one group."""
    import torch
    print("case: docs inside groups bf16 B=2 T=4096 F=512 D=256 C=256", flush=True)
    Z, V, W0 = _inputs(2, 4096, 512, 256, 1075, shared=False)
    docs = [[1280, 2048, 3328], [512, 768, 2560]]
    O, W = _run(Z, V, W0, 256, 0.01, docs, 0.0)
    _check(O, W, _oracle(Z, V, W0, 256, 0.01, docs, None), W0, TOL_BF16, "docs inside groups")
    for b in range(2):
        e = docs[b][0]
        Os, _ = ttt.chunk_scan(dev(Z[b:b + 1, :e], "bf16"), dev(V[b:b + 1, :e], "bf16"),
                               dev(W0[b], "f32"), 256, 0.01)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host_bits(O)[b, :e], host_bits(Os)[0])


def test_documents_split_wait_bound_recomputes_the_same_bits():
    """Documents inside groups and on the state chain's token split (2048), with the second
    halves' bounded wait forced to zero polls from the host: every second half gives up on the
    hand-over and recomputes its first half's tokens from W0, document resets included. The bits
    equal the run with the hand-over, and the workspace counts one event per second half."""
    import torch
    B, T, F, D, C = 2, 4096, 512, 256, 256
    print(f"case: docs bf16 B={B} T={T} F={F} D={D} C={C}, second-half wait limit 0", flush=True)
    Z, V, W0 = _inputs(B, T, F, D, 1090, shared=False)
    docs = [[1280, 2048, 3328], [512, 768, 2560]]
    Zd, Vd, W0d = dev(Z, "bf16"), dev(V, "bf16"), dev(W0, "f32")
    ws = torch.empty(ttt.lib().ttt_chunk_scan_docs_workspace(B, T, F, D, C, 1, 0.0),
                     dtype=torch.uint8, device="cuda")
    try:
        ttt.scan_test_overrides()
        O1, W1 = ttt.chunk_scan_docs(Zd, Vd, W0d, C, 0.01, doc_starts=docs, workspace=ws)
        n1 = int(ttt.chunk_scan_handover_timeouts(ws, B, T, F, D, C, torch.bfloat16).item())
        ttt.scan_test_overrides(spin_limit=0)
        O2, W2 = ttt.chunk_scan_docs(Zd, Vd, W0d, C, 0.01, doc_starts=docs, workspace=ws)
        n2 = int(ttt.chunk_scan_handover_timeouts(ws, B, T, F, D, C, torch.bfloat16).item())
        torch.cuda.synchronize()
    finally:
        ttt.scan_test_overrides()
    assert n1 == 0
    assert n2 == B * (F // 256) * (D // 256), n2
    np.testing.assert_array_equal(host_bits(O2), host_bits(O1))
    assert torch.equal(W2, W1), "W_final differs after recomputation"
    _check(O2, W2, _oracle(Z, V, W0, C, 0.01, docs, None), W0, TOL_BF16, "docs, recomputed")


def test_documents_inside_groups_small_chunks_and_fp32_out():
    """64-token chunks (16 per group, per-element correction masks): starts at offsets 256 and
    768 inside groups and one at a group start; fp32 output, shared W0, eta < 0."""
    print("case: docs inside groups bf16 B=1 T=3000 F=256 D=128 C=64", flush=True)
    Z, V, W0 = _inputs(1, 3000, 256, 128, 1076)
    docs = [[256, 1792, 2048]]
    O, W = _run(Z, V, W0, 64, -0.01, docs, 0.0, out_dtype="f32")
    _check(O, W, _oracle(Z, V, W0, 64, -0.01, docs, None), W0, TOL_BF16,
           "docs inside groups, C=64")


def test_documents_inside_groups_with_clipping():
    print("case: docs inside groups + clip bf16 B=1 T=3584 F=512 D=256 C=512", flush=True)
    Z, V, W0 = _inputs(1, 3584, 512, 256, 1077)
    docs = [[1536, 2560]]
    tau = _median_tau(Z, V, 512, 0.01)
    O, W = _run(Z, V, W0, 512, 0.01, docs, tau)
    _check(O, W, _oracle(Z, V, W0, 512, 0.01, docs, tau), W0, TOL_BF16,
           "docs inside groups + clip")


def test_documents_on_group_boundaries_with_clipping():
    print("case: docs on group boundaries + clip bf16 B=1 T=3072 F=512 D=256 C=256", flush=True)
    Z, V, W0 = _inputs(1, 3072, 512, 256, 1080)
    docs = [[2048]]
    tau = _median_tau(Z, V, 256, 0.01)
    O, W = _run(Z, V, W0, 256, 0.01, docs, tau, out_dtype="f32")
    _check(O, W, _oracle(Z, V, W0, 256, 0.01, docs, tau), W0, TOL_BF16, "docs on groups + clip")


def test_bench_workload_documents_and_clipping_sampled():
    """T=32768, C=512, d_model=2560, d_ff=9728, eta=1e-4, documents at 8192 (a group start) and
    20992 (inside a group), clipping at the median chunk norm: sampled rows against the
    exclusive-prefix oracle run on each document with the targets scaled by the exact clip
    factors."""
    import torch
    print("case: docs+clip bf16 T=32768 C=512 D=2560 F=9728 (generating inputs)", flush=True)
    inp = gen.inplace_mlp(32768, 2560, 9728, 512, eta=1e-4, seed_base=20)
    z = gen.bf16_bits_to_f32(inp.Z[0])
    v = gen.bf16_bits_to_f32(inp.V[0])
    norms = od.delta_norms_gram(z, v, 512, 1e-4)
    tau = float(np.median(norms))
    scale = np.minimum(1.0, tau / norms)
    docs = [8192, 20992]
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    O, W = ttt.chunk_scan_docs(Z, V, W0, 512, 1e-4, doc_starts=[docs], clip_tau=tau)
    torch.cuda.synchronize()
    vs = v * np.repeat(scale, 512)[:, None].astype(np.float32)
    bounds = [0] + docs + [32768]
    rng = np.random.default_rng(1)
    for s, e in zip(bounds[:-1], bounds[1:]):
        rows = np.unique(np.concatenate([[s, s + 511, s + 512, e - 1],
                                         rng.integers(s, e, 12)]))
        ref = oi.prefix_rows(z[s:e], vs[s:e], inp.W0, 512, 1e-4, rows - s)
        got = host_f64(O[0, torch.as_tensor(rows, device=O.device)])
        assert_close(got, ref, TOL_BF16, f"sampled O rows of document [{s}, {e})")
    dm = np.array([0, 3, 1280, 2559])
    wref = oi.final_state_rows(z[20992:], vs[20992:], inp.W0, 1e-4, dm)
    got = host_f64(W[0, torch.as_tensor(dm, device=W.device)])
    assert_close(got - inp.W0[dm], wref - inp.W0[dm], TOL_BF16, "sampled W_final - W0")
