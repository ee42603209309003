"""GPU parity of ttt_linear_minibatch against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.ttt_linear as ol
from helpers import TOL_BF16, TOL_F32, assert_close, dev, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _oracle(inp, b, eta, W0=None):
    return ol.minibatch_gd_batched(inp.f64("Q"), inp.f64("K"), inp.f64("V"), W0, b, eta)


def _run(inp, b, eta, W0=None, out_dtype=None):
    import torch
    od = None if out_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    O, W, L = ttt.linear_minibatch(dev(inp.Q, inp.dtype), dev(inp.K, inp.dtype),
                                   dev(inp.V, inp.dtype), b, eta,
                                   W0=None if W0 is None else dev(W0, "f32"), out_dtype=od)
    torch.cuda.synchronize()
    return host_f64(O), host_f64(W), host_f64(L)


@pytest.mark.parametrize("b", [16, 32, 48, 64])
def test_bf16_matrix_core_kernel(b):
    print(f"case: bf16 B=2 T=384 H=4 b={b} eta=0.1", flush=True)
    inp = gen.ttt_linear_inputs(2, 384, 256, 4, 64, seed_base=500)
    O, W, L = _run(inp, b, 0.1)
    Oref, Wref, Lref = _oracle(inp, b, 0.1)
    assert_close(O, Oref, TOL_BF16, "O")
    assert_close(W, Wref, TOL_BF16, "W_final")
    assert_close(L, Lref, TOL_BF16, "loss")


@pytest.mark.parametrize("b,T", [(16, 400), (32, 416), (16, 64), (32, 64), (64, 64)])
def test_bf16_chunked_and_per_minibatch_paths(b, T):
    # T a multiple of 64 runs in 64-token chunks, other T one mini-batch per step; both against
    # the oracle, with an initial state and fp32 outputs
    print(f"case: bf16 B=2 T={T} H=3 b={b} eta=0.1 W0", flush=True)
    inp = gen.ttt_linear_inputs(2, T, 192, 3, 64, seed_base=505)
    W0 = (np.random.default_rng(3).standard_normal((2, 3, 64, 64)) * 0.05).astype(np.float32)
    O, W, L = _run(inp, b, 0.1, W0=W0, out_dtype="f32")
    Oref, Wref, Lref = _oracle(inp, b, 0.1, W0=W0.astype(np.float64))
    assert_close(O, Oref, TOL_BF16, "O")
    assert_close(W, Wref, TOL_BF16, "W_final")
    assert_close(L, Lref, TOL_BF16, "loss")


def test_bf16_with_initial_state_fp32_out():
    inp = gen.ttt_linear_inputs(1, 256, 128, 2, 64, seed_base=510)
    W0 = (np.random.default_rng(1).standard_normal((1, 2, 64, 64)) * 0.05).astype(np.float32)
    O, W, L = _run(inp, 16, 0.1, W0=W0, out_dtype="f32")
    Oref, Wref, Lref = _oracle(inp, 16, 0.1, W0=W0.astype(np.float64))
    assert_close(O, Oref, TOL_BF16, "O")
    assert_close(W, Wref, TOL_BF16, "W_final")
    assert_close(L, Lref, TOL_BF16, "loss")


@pytest.mark.parametrize("b", [1, 4, 16])
def test_small_minibatch_is_delta_rule_region(b):
    # Stable tiny case (K, Q scaled by 1/8, eta = 0.5): b = 1 is the delta rule.
    inp = gen.ttt_linear_inputs(2, 256, 128, 4, 64, seed_base=520, qk_scale=0.125)
    O, W, L = _run(inp, b, 0.5)
    Oref, Wref, Lref = _oracle(inp, b, 0.5)
    assert_close(O, Oref, TOL_BF16, "O")
    assert_close(W, Wref, TOL_BF16, "W_final")
    if b == 1:
        Od, Wd = zip(*[ol.delta_rule(inp.f64("Q")[i], inp.f64("K")[i], inp.f64("V")[i], None,
                                     0.5) for i in range(2)])
        assert_close(O, np.stack(Od), TOL_BF16, "O vs delta rule")


@pytest.mark.parametrize("b", [1, 16, 64])
def test_fp32_path(b):
    inp = gen.ttt_linear_inputs(1, 128, 128, 2, 64, seed_base=530, dtype="f32", qk_scale=0.25)
    O, W, L = _run(inp, b, 0.3)
    Oref, Wref, Lref = _oracle(inp, b, 0.3)
    assert_close(O, Oref, TOL_F32, "O")
    assert_close(W, Wref, TOL_F32, "W_final")
    assert_close(L, Lref, TOL_F32, "loss")


def test_eta_zero():
    inp = gen.ttt_linear_inputs(1, 128, 128, 2, 64, seed_base=540)
    W0 = (np.random.default_rng(2).standard_normal((1, 2, 64, 64)) * 0.1).astype(np.float32)
    O, W, _ = _run(inp, 16, 0.0, W0=W0)
    np.testing.assert_array_equal(W, W0)
    assert_close(O, np.einsum("bthd,bhde->bthe", inp.f64("Q"), W0.astype(np.float64)),
                 TOL_BF16, "O = Q W0")


def test_bench_workload():
    """B=8, T=8192, d_model=2048, 32 heads x 64, b=16, eta=0.1, bf16 -- sampled heads."""
    print("case: bf16 B=8 T=8192 H=32 b=16 (generating inputs)", flush=True)
    inp = gen.ttt_linear_inputs(8, 8192, 2048, 32, 64, seed_base=40)
    O, W, L = _run(inp, 16, 0.1)
    for b, h in [(0, 0), (3, 17), (7, 31)]:
        o, w, l = ol.minibatch_gd(inp.f64("Q")[b][:, h:h + 1], inp.f64("K")[b][:, h:h + 1],
                                  inp.f64("V")[b][:, h:h + 1], None, 16, 0.1)
        assert_close(O[b][:, h], o[:, 0], TOL_BF16, f"O[b={b},h={h}]")
        assert_close(W[b][h], w[0], TOL_BF16, f"W[b={b},h={h}]")
        assert_close(L[b][:, h], l[:, 0], TOL_BF16, f"loss[b={b},h={h}]")
