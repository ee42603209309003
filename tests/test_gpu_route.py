"""GPU parity of ttt_surprisal_route: routing decisions are compared bit for bit with the oracle
fed the same fp32 losses, on hand-built cases, on the SR-TTT workload end to end, on odd chunk
sizes and with a forced ring overflow."""
import json
import os

import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.route as orr
import oracle.ttt_linear as ol
from helpers import dev, host_bits, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _gpu_route(loss_f32, K, V, kv_dtype, chunk, **kw):
    import torch
    out = ttt.surprisal_route(dev(loss_f32, "f32"), dev(K, kv_dtype), dev(V, kv_dtype), chunk,
                              **kw)
    torch.cuda.synchronize()
    return {k: (None if v is None else host_bits(v)) for k, v in out.items()}


def _compare(got, ref, kv=True):
    np.testing.assert_array_equal(got["tau"], ref["tau"])
    np.testing.assert_array_equal(got["mask"], ref["mask"])
    np.testing.assert_array_equal(got["idx"], ref["idx"])
    np.testing.assert_array_equal(got["count"], ref["count"])
    np.testing.assert_array_equal(got["total"], ref["total"])
    if kv:
        np.testing.assert_array_equal(got["k"], ref["k"].reshape(got["k"].shape))
        np.testing.assert_array_equal(got["v"], ref["v"].reshape(got["v"].shape))


def test_hand_cases(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "route_hand.json")))
    p = g["params"]
    for c in g["cases"]:
        L = np.array(c["L"], np.float32)[None, :, None]           # B=1, H=1
        T = L.shape[1]
        K = np.arange(T * 8, dtype=np.uint16).reshape(1, T, 8)
        out = _gpu_route(L, K, K, "bf16", c["chunk"], pct=p["pct"], ema=p["ema"],
                         ratio=p["ratio"], capacity=c["capacity"])
        assert np.flatnonzero(out["mask"][0]).tolist() == c["routed"], c["name"]
        assert int(out["total"][0]) == c["total"], c["name"]
        if c["tau"] is not None:
            assert out["tau"][0].tolist() == c["tau"], c["name"]
        if "slots" in c:
            assert out["idx"][0].tolist() == c["slots"], c["name"]
        ref = orr.surprisal_route(L, K, K, c["chunk"], p["pct"], p["ema"], p["ratio"],
                                  c["capacity"])
        _compare(out, ref)


def _sr_workload():
    inp = gen.route_inputs(B=4, T=2048, d_model=1024, H=16, dh=64, seed_base=50)
    return inp


def test_sr_workload_end_to_end():
    """B=4, T=2048, 16 heads x 64, chunk 64, TTT-Linear b=64 eta=0.01; capacity 256."""
    import torch
    inp = _sr_workload()
    Q, K, V = dev(inp.Q, "bf16"), dev(inp.K, "bf16"), dev(inp.V, "bf16")
    _, _, loss = ttt.linear_minibatch(Q, K, V, 64, 0.01)
    out = ttt.surprisal_route(loss, K, V, 64)
    torch.cuda.synchronize()
    got = {k: host_bits(v) for k, v in out.items()}
    L = host_bits(loss)
    # 1. decisions are bit-exact given the same losses
    ref = orr.surprisal_route(L, inp.K, inp.V, 64)
    _compare(got, ref)
    # 2. against the oracle's own fp64 losses rounded to fp32: tokens whose loss lies within
    #    1e-4 (relative) of either side's threshold may legitimately differ; all others agree.
    _, _, Lo = ol.minibatch_gd_batched(inp.f64("Q"), inp.f64("K"), inp.f64("V"), None, 64, 0.01)
    ref2 = orr.surprisal_route(Lo.astype(np.float32), inp.K, inp.V, 64)
    Lg = np.stack([orr.head_sum(L[b]) for b in range(4)])
    Lr = np.stack([orr.head_sum(Lo[b].astype(np.float32)) for b in range(4)])
    tg = np.repeat(got["tau"], 64, axis=1)
    tr = np.repeat(ref2["tau"], 64, axis=1)
    band = (np.abs(Lg - tg) <= 1e-4 * tg) | (np.abs(Lr - tr) <= 1e-4 * tr)
    differ = got["mask"] != ref2["mask"]
    print(f"  routed per sequence: {got['total'].tolist()} (oracle losses: "
          f"{ref2['total'].tolist()}); tokens in the tie band: {int(band.sum())}; "
          f"decisions that differ: {int(differ.sum())}", flush=True)
    assert not (differ & ~band).any()
    np.testing.assert_allclose(got["tau"], ref2["tau"], rtol=1e-3)
    outliers = inp.meta["outliers"]
    for b in range(4):
        assert got["mask"][b, outliers[b]].any()


@pytest.mark.parametrize("chunk,cap", [(48, 256), (100, 64), (128, 16), (1, 8), (1024, 300)])
def test_odd_chunks_and_overflow(chunk, cap):
    rng = np.random.default_rng(chunk)
    T = 4096 // chunk * chunk if chunk > 1 else 512
    L = rng.exponential(1.0, (3, T, 5)).astype(np.float32)
    L[:, rng.choice(T, max(1, T // 40), replace=False)] *= 50.0
    K = rng.integers(0, 65535, (3, T, 5 * 8)).astype(np.uint16)
    V = rng.integers(0, 65535, (3, T, 5 * 8)).astype(np.uint16)
    got = _gpu_route(L, K, V, "bf16", chunk, capacity=cap)
    ref = orr.surprisal_route(L, K, V, chunk, capacity=cap)
    _compare(got, ref)


@pytest.mark.parametrize("chunk,pct", [(37, 0.95), (64, 0.95), (64, 0.5), (37, 0.6), (64, 0.89),
                                       (128, 0.95), (512, 0.95)])
def test_ties_and_negative_losses(chunk, pct):
    # integer-valued per-head losses (many ties, some negative sums): the percentile is a value of
    # the chunk whichever method picks it: repeated maxima when it lies within 8 values of the
    # top of a chunk of at most 64 (the 95th percentile; 0.89 of 64 is the 8th largest), rank
    # counting below that (0.5, 0.6), the radix select past 64 values
    rng = np.random.default_rng(700 + chunk + int(100 * pct))
    T = 2048 // chunk * chunk
    L = rng.integers(-2, 6, (2, T, 8)).astype(np.float32)
    K = rng.integers(0, 65535, (2, T, 8 * 8)).astype(np.uint16)
    V = rng.integers(0, 65535, (2, T, 8 * 8)).astype(np.uint16)
    got = _gpu_route(L, K, V, "bf16", chunk, pct=pct, capacity=40)
    ref = orr.surprisal_route(L, K, V, chunk, pct, capacity=40)
    _compare(got, ref)


@pytest.mark.parametrize("T,chunk,cap", [(24576, 64, 256), (12288, 1024, 300), (3000, 1, 40),
                                         (17408, 128, 4096)])
def test_long_sequences_in_windows(T, chunk, cap):
    # sequences longer than one window (8192 tokens, or 1024 chunks): the threshold and the
    # routed count carry across windows, the ring fills across them; 2% outliers keep routing
    # busy, and a capacity of 4096 spans several windows' routed tokens
    print(f"case: route T={T} chunk={chunk} capacity={cap} (windows)", flush=True)
    rng = np.random.default_rng(T + chunk)
    L = rng.gamma(2.0, 1.0, (2, T, 4)).astype(np.float32)
    out = rng.random((2, T)) < 0.02
    L[out] *= np.float32(8.0)
    K = rng.integers(0, 65535, (2, T, 4 * 8)).astype(np.uint16)
    V = rng.integers(0, 65535, (2, T, 4 * 8)).astype(np.uint16)
    # chunk ratio 0.5: 600-1100 tokens routed per sequence, past every capacity but 4096
    got = _gpu_route(L, K, V, "bf16", chunk, ratio=0.5, capacity=cap)
    ref = orr.surprisal_route(L, K, V, chunk, ratio=0.5, capacity=cap)
    print(f"  routed per sequence: {ref['total'].tolist()}", flush=True)
    assert ref["total"].min() > 500
    _compare(got, ref)


def test_fp32_rows_and_other_thresholds():
    rng = np.random.default_rng(9)
    L = rng.gamma(2.0, 1.0, (2, 1024, 3)).astype(np.float32)
    K = rng.standard_normal((2, 1024, 3 * 4)).astype(np.float32)
    V = rng.standard_normal((2, 1024, 3 * 4)).astype(np.float32)
    for pct, ema, ratio in [(0.5, 0.5, 0.5), (1.0, 0.0, 0.1), (0.9, 0.99, 1.0)]:
        got = _gpu_route(L, K, V, "f32", 32, pct=pct, ema=ema, ratio=ratio, capacity=100)
        ref = orr.surprisal_route(L, K, V, 32, pct, ema, ratio, 100)
        _compare(got, ref)


def test_reused_outputs_match_fresh_outputs():
    """Routing into the tensors of an earlier call (out=) gives the same results as a fresh call."""
    import torch
    rng = np.random.default_rng(5)
    L = rng.exponential(1.0, (2, 1024, 4)).astype(np.float32)
    L[:, rng.choice(1024, 30, replace=False)] *= 40.0
    K = rng.integers(0, 65535, (2, 1024, 4 * 8)).astype(np.uint16)
    V = rng.integers(0, 65535, (2, 1024, 4 * 8)).astype(np.uint16)
    Ld, Kd, Vd = dev(L, "f32"), dev(K, "bf16"), dev(V, "bf16")
    first = ttt.surprisal_route(Ld, Kd, Vd, 64, capacity=48)
    L2 = L.copy()
    L2[:, 512:] *= 3.0                     # different decisions on the second call
    again = ttt.surprisal_route(dev(L2, "f32"), Kd, Vd, 64, capacity=48, out=first)
    fresh = ttt.surprisal_route(dev(L2, "f32"), Kd, Vd, 64, capacity=48)
    torch.cuda.synchronize()
    assert again is first
    for k in fresh:
        np.testing.assert_array_equal(host_bits(again[k]), host_bits(fresh[k]))
    _compare({k: host_bits(v) for k, v in again.items()},
             orr.surprisal_route(L2, K, V, 64, capacity=48))
