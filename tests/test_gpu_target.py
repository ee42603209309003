"""GPU parity of ttt_lm_target (the LM-aligned target producer) against the fp64 oracle."""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.target as ot
from helpers import TOL_BF16, assert_close, dev, host_bits, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(B, T, din, dout, width, seed):
    X0 = gen.f32_to_bf16_bits(gen.normal(seed, (B, T, din)))
    cw = gen.normal(seed + 1, (width, din), 0.5)
    W = gen.f32_to_bf16_bits(gen.normal(seed + 2, (din, dout), 1.0 / np.sqrt(din)))
    return X0, cw, W


def _run(X0, cw, W, chunk, out_dtype=None):
    import torch
    od = None if out_dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[out_dtype]
    V = ttt.lm_target(dev(X0, "bf16"), dev(cw, "f32"), dev(W, "bf16"), chunk, out_dtype=od)
    torch.cuda.synchronize()
    return V


def _oracle(X0, cw, W, chunk):
    return ot.lm_target_batched(gen.bf16_bits_to_f32(X0), cw, gen.bf16_bits_to_f32(W), chunk)


@pytest.mark.parametrize("B,T,din,dout,chunk,width", [
    (2, 1000, 128, 96, 100, 4),     # ragged token tiles, one partial output tile
    (1, 777, 192, 272, 64, 5),      # the page's kernel size 5; output tiles 256 + 16
    (1, 512, 64, 16, 512, 1),       # one chunk, next token only
    (2, 300, 128, 128, 7, 3),       # chunk not a multiple of anything
])
def test_parity(B, T, din, dout, chunk, width):
    print(f"case: target B={B} T={T} d_in={din} d_out={dout} chunk={chunk} width={width}",
          flush=True)
    X0, cw, W = _inputs(B, T, din, dout, width, 700 + T)
    V = _run(X0, cw, W, chunk)
    assert_close(host_f64(V), _oracle(X0, cw, W, chunk), TOL_BF16, "V_hat")


def test_fp32_output_and_chunk_one_is_zero():
    X0, cw, W = _inputs(1, 256, 128, 64, 4, 720)
    V = _run(X0, cw, W, 64, out_dtype="f32")
    assert V.element_size() == 4
    assert_close(host_f64(V), _oracle(X0, cw, W, 64), TOL_BF16, "V_hat fp32")
    Z = _run(X0, cw, W, 1)                  # every token is the end of its own chunk
    assert not host_bits(Z).any()


def test_no_row_of_a_later_chunk_is_read():
    # bit-identical targets for chunks <= i when every row of chunks > i changes
    X0, cw, W = _inputs(1, 1024, 128, 128, 4, 730)
    V1 = host_bits(_run(X0, cw, W, 256))
    for i in (0, 2):
        X1 = X0.copy()
        X1[0, (i + 1) * 256:] ^= np.uint16(0x0100)
        V2 = host_bits(_run(X1, cw, W, 256))
        np.testing.assert_array_equal(V1[0, :(i + 1) * 256], V2[0, :(i + 1) * 256])
        assert (V1[0, (i + 1) * 256:] != V2[0, (i + 1) * 256:]).any()


def test_bench_shape_sampled_rows():
    """T=32768, d_model=2560, chunk 512, width 4 (the scan workload's target): sampled rows."""
    import torch
    print("case: target T=32768 d=2560 (generating inputs)", flush=True)
    T, d, C = 32768, 2560, 512
    X0 = gen.f32_to_bf16_bits(gen.normal(24, (1, T, d)))
    cw = gen.normal(25, (4, d), 0.5)
    W = gen.f32_to_bf16_bits(gen.normal(26, (d, d), 1.0 / np.sqrt(d)))
    V = _run(X0, cw, W, C)
    rows = [0, 1, 507, 508, 511, 512, 1023, 16384, 32763, 32767]
    ref = ot.lm_target_rows(gen.bf16_bits_to_f32(X0[0]), cw, gen.bf16_bits_to_f32(W), C, rows)
    got = host_f64(V[0, torch.as_tensor(rows, device=V.device)])
    assert_close(got, ref, TOL_BF16, "sampled V_hat rows")
    assert not host_bits(V[0, torch.as_tensor([511, 32767], device=V.device)]).any()
