"""Seeded random sweeps against the fp64 oracle: the bf16 scan entry points over shapes drawn
across the masked and unmasked paths (ragged T, chunk sizes that are and are not whole 32-token
steps, d_model off the 256-tile grid), shared and per-sequence W0, negative eta, random document
starts and clipping; and TTT-Linear over random sizes and mini-batch sizes (all three kernels),
followed by routing on its loss, bit for bit; and the LM-aligned target producer over random
widths, chunks and sizes."""
import random

import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.docs as od
import oracle.inplace as oi
from helpers import TOL_BF16, assert_close, dev, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _draw(rng, big):
    if big:
        F, D = rng.choice([256, 512, 768]), rng.choice([256, 272, 512])
        C = rng.choice([128, 256, 512, 1024])
        T = rng.choice([C * rng.randint(2, 12), rng.randint(2048, 8192)])
    else:
        F, D = rng.choice([64, 128, 192, 256, 320, 512]), rng.choice([16, 48, 64, 128, 256, 272])
        C = rng.choice([16, 32, 64, 100, 128, 256, 512])
        T = rng.choice([C * rng.randint(1, 9), rng.randint(1, 2500)])
    return F, D, C, T, rng.choice([1, 1, 2]), rng.choice([3e-3, -2e-3, 1e-2]), rng.random() < 0.6


@pytest.mark.parametrize("case", [("small", s) for s in range(8)] + [("big", s) for s in range(6)])
def test_random_shapes(case):
    mode, seed = case
    rng = random.Random(1000 * (mode == "big") + seed)
    F, D, C, T, B, eta, shared = _draw(rng, mode == "big")
    docs = rng.random() < 0.3
    clip = rng.random() < 0.3
    inp = gen.inplace_mlp(T, D, F, C, eta=eta, B=B, seed_base=700 + seed + 50 * (mode == "big"),
                          shared_w0=shared)
    starts, tau = None, 0.0
    if docs:
        cand = list(range(C, T, C))
        starts = [sorted(rng.sample(cand, min(len(cand), rng.randint(0, 3)))) for _ in range(B)]
    if clip:
        tau = float(np.median(np.concatenate(
            [od.delta_norms(inp.z_f64(b), inp.v_f64(b), C, eta) for b in range(B)])))
    print(f"case: {mode} {seed}: B={B} T={T} C={C} D={D} F={F} eta={eta} shared={shared} "
          f"docs={starts} tau={tau:.3g}", flush=True)
    import torch
    Z, V, W0 = dev(inp.Z, "bf16"), dev(inp.V, "bf16"), dev(inp.W0, "f32")
    if docs or clip:
        O, W = ttt.chunk_scan_docs(Z, V, W0, C, eta, doc_starts=starts, clip_tau=tau)
    else:
        O, W = ttt.chunk_scan(Z, V, W0, C, eta)
    torch.cuda.synchronize()
    Oh, Wh = host_f64(O), host_f64(W)
    for b in range(B):
        w0 = inp.w0_f64(b)
        if docs or clip:
            o, w = od.chunk_scan_docs(inp.z_f64(b), inp.v_f64(b), w0, C, eta,
                                      starts[b] if starts else (), tau if clip else None)
        else:
            o, w = oi.chunk_scan(inp.z_f64(b), inp.v_f64(b), w0, C, eta)
        assert_close(Oh[b], o, TOL_BF16, f"O[{b}]")
        assert_close(Wh[b] - w0, w - w0, TOL_BF16, f"W_final - W0 [{b}]")


@pytest.mark.parametrize("seed", range(8))
def test_random_linear_then_route(seed):
    """TTT-Linear at random sizes, mini-batch sizes and initial states, then routing on its loss
    (decisions, thresholds and cache bit for bit against the oracle fed the same loss)."""
    import oracle.route as orr
    import oracle.ttt_linear as ol
    rng = random.Random(2000 + seed)
    B, H = rng.choice([1, 2, 3]), rng.choice([1, 2, 4, 8])
    rc = rng.choice([64, 128])
    T = rc * rng.randint(2, 12)
    b = rng.choice([x for x in (1, 4, 8, 16, 32, 48, 64) if T % x == 0])
    eta = rng.choice([0.05, 0.1])
    with_w0 = rng.random() < 0.5
    cap = rng.choice([8, 64, 256])
    print(f"case: linear+route B={B} T={T} H={H} b={b} eta={eta} W0={with_w0} chunk={rc} "
          f"capacity={cap}", flush=True)
    inp = gen.ttt_linear_inputs(B, T, 64 * H, H, 64, seed_base=900 + 10 * seed, qk_scale=0.5)
    W0 = (np.random.default_rng(seed).standard_normal((B, H, 64, 64)) * 0.02).astype(np.float32) \
        if with_w0 else None
    import torch
    O, W, L = ttt.linear_minibatch(dev(inp.Q, "bf16"), dev(inp.K, "bf16"), dev(inp.V, "bf16"), b,
                                   eta, W0=None if W0 is None else dev(W0, "f32"))
    route = ttt.surprisal_route(L, dev(inp.K, "bf16"), dev(inp.V, "bf16"), rc, capacity=cap)
    torch.cuda.synchronize()
    o, w, l = ol.minibatch_gd_batched(inp.f64("Q"), inp.f64("K"), inp.f64("V"),
                                      None if W0 is None else W0.astype(np.float64), b, eta)
    assert_close(host_f64(O), o, TOL_BF16, "O")
    assert_close(host_f64(W), w, TOL_BF16, "W_final")
    assert_close(host_f64(L), l, TOL_BF16, "loss")
    ref = orr.surprisal_route(L.cpu().numpy(), inp.K, inp.V, rc, capacity=cap)
    for k in ("tau", "mask", "idx", "count", "total"):
        np.testing.assert_array_equal(route[k].cpu().numpy(), ref[k], err_msg=k)


@pytest.mark.parametrize("seed", range(6))
def test_random_target_producer(seed):
    """The LM-aligned target at random sizes: widths up to 16, chunks from 1 token to more than T,
    T off the 64-token tiles, d_out off the 256-column tiles, both output types."""
    import oracle.target as ot
    rng = random.Random(3000 + seed)
    B, T = rng.choice([1, 2]), rng.choice([rng.randint(1, 80), rng.randint(100, 1500)])
    din, dout = 64 * rng.randint(1, 5), 16 * rng.randint(1, 20)
    chunk, width = rng.choice([1, 2, 13, 64, 100, 4096]), rng.randint(1, 16)
    out = rng.choice(["bf16", "f32"])
    print(f"case: target B={B} T={T} d_in={din} d_out={dout} chunk={chunk} width={width} out={out}",
          flush=True)
    X0 = gen.f32_to_bf16_bits(gen.normal(4000 + seed, (B, T, din)))
    cw = gen.normal(4100 + seed, (width, din), 0.5)
    W = gen.f32_to_bf16_bits(gen.normal(4200 + seed, (din, dout), 1.0 / np.sqrt(din)))
    import torch
    V = ttt.lm_target(dev(X0, "bf16"), dev(cw, "f32"), dev(W, "bf16"), chunk,
                      out_dtype={"f32": torch.float32, "bf16": torch.bfloat16}[out])
    torch.cuda.synchronize()
    ref = ot.lm_target_batched(gen.bf16_bits_to_f32(X0), cw, gen.bf16_bits_to_f32(W), chunk)
    assert_close(host_f64(V), ref, TOL_BF16, "V_hat")
