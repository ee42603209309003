"""GPU parity of ttt_gated_z (the gated-MLP activation that feeds the chunk scan) against the
fp64 oracle."""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.mlp as om
from helpers import TOL_BF16, assert_close, dev, host_bits, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(B, T, dm, dff, seed):
    X = gen.f32_to_bf16_bits(gen.normal(seed, (B, T, dm)))
    Wg = gen.f32_to_bf16_bits(gen.normal(seed + 1, (dm, dff), 1.0 / np.sqrt(dm)))
    Wu = gen.f32_to_bf16_bits(gen.normal(seed + 2, (dm, dff), 1.0 / np.sqrt(dm)))
    return X, Wg, Wu


def _run(X, Wg, Wu, out_dtype=None):
    import torch
    od = None if out_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    W = np.ascontiguousarray(np.concatenate([Wg.T, Wu.T], axis=0))  # [2 d_ff, d_model]
    Z = ttt.gated_z(dev(X, "bf16"), dev(W, "bf16"), out_dtype=od)
    torch.cuda.synchronize()
    return Z


def _oracle(X, Wg, Wu):
    f = gen.bf16_bits_to_f32
    return np.stack([om.gated_z(f(x), f(Wg), f(Wu)) for x in X])


@pytest.mark.parametrize("B,T,dm,dff", [
    (2, 1000, 128, 96),     # ragged token tile, one partial column block
    (1, 777, 192, 272),     # column blocks 128 + 128 + 16, three K steps
    (1, 128, 64, 8),        # one K step, the narrowest d_ff
    (3, 300, 256, 384),     # several sequences, whole column blocks, ragged tokens
    (1, 1, 64, 128),        # one token
])
def test_parity(B, T, dm, dff):
    print(f"case: gated_z B={B} T={T} d_model={dm} d_ff={dff}", flush=True)
    X, Wg, Wu = _inputs(B, T, dm, dff, 800 + T)
    Z = _run(X, Wg, Wu)
    assert Z.shape == (B, T, dff)
    assert_close(host_f64(Z), _oracle(X, Wg, Wu), TOL_BF16, "Z")


def test_fp32_output():
    X, Wg, Wu = _inputs(1, 640, 128, 256, 830)
    Z = _run(X, Wg, Wu, out_dtype="f32")
    assert Z.element_size() == 4
    assert_close(host_f64(Z), _oracle(X, Wg, Wu), 1e-4, "Z fp32")


def test_zero_gate_or_up_gives_exact_zero():
    # SiLU(0) = 0: a zero gate projection zeroes Z (up to the sign of zero) whatever the up
    # projection, and so does a zero up projection
    X, Wg, Wu = _inputs(1, 256, 128, 128, 840)
    assert not (host_bits(_run(X, np.zeros_like(Wg), Wu)) & 0x7FFF).any()
    assert not (host_bits(_run(X, Wg, np.zeros_like(Wu))) & 0x7FFF).any()


def test_gate_and_up_halves_are_not_swapped():
    # Z(Wg, Wu) matches the oracle and differs clearly from the oracle with the roles swapped
    X, Wg, Wu = _inputs(1, 256, 128, 128, 845)
    got = host_f64(_run(X, Wg, Wu))[0]
    f = gen.bf16_bits_to_f32
    swapped = om.gated_z(f(X[0]), f(Wu), f(Wg))
    assert np.linalg.norm(got - swapped) > 0.3 * np.linalg.norm(swapped)


def test_rows_are_independent_and_batches_do_not_mix():
    X, Wg, Wu = _inputs(2, 384, 128, 256, 850)
    Z1 = host_bits(_run(X, Wg, Wu))
    X2 = X.copy()
    X2[1, 200] ^= np.uint16(0x0100)
    Z2 = host_bits(_run(X2, Wg, Wu))
    diff = np.argwhere((Z1 != Z2).any(axis=2))
    assert diff.tolist() == [[1, 200]]


def test_bench_shape_sampled_rows():
    """T=32768, d_model=2560, d_ff=9728 (the scan workload's Z): sampled rows."""
    import torch
    print("case: gated_z T=32768 d_model=2560 d_ff=9728 (generating inputs)", flush=True)
    T, dm, dff = 32768, 2560, 9728
    X = gen.f32_to_bf16_bits(gen.normal(21, (1, T, dm)))
    Wg = gen.f32_to_bf16_bits(gen.normal(22, (dm, dff), 1.0 / np.sqrt(dm)))
    Wu = gen.f32_to_bf16_bits(gen.normal(23, (dm, dff), 1.0 / np.sqrt(dm)))
    Z = _run(X, Wg, Wu)
    rows = [0, 1, 127, 128, 4095, 16384, 32766, 32767]
    f = gen.bf16_bits_to_f32
    ref = om.gated_z_rows(f(X[0]), f(Wg), f(Wu), rows)
    got = host_f64(Z[0, torch.as_tensor(rows, device=Z.device)])
    assert_close(got, ref, TOL_BF16, "sampled Z rows")
