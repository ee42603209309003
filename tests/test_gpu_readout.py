"""GPU parity of ttt_cache_readout (SR residual-cache attention with alpha fusion) against the fp64
oracle: the attention part alone and fused, both output types, in place, the empty cache, FIFO
eviction, causality, and the SR-TTT workload end to end (TTT-Linear -> routing -> readout)."""
import numpy as np
import pytest

import chunked_weight_sequence_amd as ttt
import gen
import oracle.readout as orr
from helpers import TOL_BF16, assert_close, dev, host_bits, host_f64, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(B, T, H, seed, density, out_dtype="bf16"):
    rng = np.random.default_rng(seed)
    HD = H * 64
    Q, K, V = (gen.f32_to_bf16_bits(rng.standard_normal((B, T, HD)).astype(np.float32))
               for _ in range(3))
    O = rng.standard_normal((B, T, HD)).astype(np.float32)
    if out_dtype == "bf16":
        O = gen.f32_to_bf16_bits(O)
    routed = (rng.random((B, T)) < density).astype(np.uint8)
    alpha = rng.uniform(-0.5, 1.5, HD).astype(np.float32)
    return Q, K, V, O, routed, alpha


def _f(a):
    return gen.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def _run(Q, K, V, O, routed, alpha, H, chunk, cap, scale=0.125, out_dtype="bf16", inplace=False):
    import torch
    Od = dev(O, out_dtype)
    out = ttt.cache_readout(dev(Q, "bf16"), dev(K, "bf16"), dev(V, "bf16"),
                            torch.from_numpy(routed).cuda(), Od, dev(alpha, "f32"), H, chunk, cap,
                            scale, out=Od if inplace else None)
    torch.cuda.synchronize()
    if inplace:
        assert out.data_ptr() == Od.data_ptr()
    return out


def _oracle(Q, K, V, O, routed, alpha, H, chunk, cap, scale=0.125):
    return orr.cache_readout(_f(Q), _f(K), _f(V), routed, _f(O), alpha, H, chunk, cap, scale)


@pytest.mark.parametrize("B,T,H,chunk,cap,density", [
    (2, 512, 4, 64, 32, 0.2),      # cache saturates: eviction from the fourth chunk on
    (1, 640, 2, 128, 256, 0.5),    # two 64-token blocks per chunk, cache up to full
    (3, 256, 1, 64, 1, 0.3),       # capacity one
    (1, 1024, 3, 256, 17, 0.05),   # sparse routing, ragged cache blocks
])
def test_attention_part_and_fused_output(B, T, H, chunk, cap, density):
    print(f"case: readout B={B} T={T} H={H} chunk={chunk} cap={cap} density={density}",
          flush=True)
    Q, K, V, O, routed, alpha = _inputs(B, T, H, 900 + T, density)
    zeros, ones = np.zeros(O.shape, np.float32), np.ones(H * 64, np.float32)
    att = _run(Q, K, V, zeros, routed, ones, H, chunk, cap, out_dtype="f32")
    assert_close(host_f64(att), _oracle(Q, K, V, zeros, routed, ones, H, chunk, cap),
                 TOL_BF16, "attention")
    got = _run(Q, K, V, O, routed, alpha, H, chunk, cap)
    assert_close(host_f64(got), _oracle(Q, K, V, O, routed, alpha, H, chunk, cap), TOL_BF16,
                 "fused output")


def test_fp32_output_in_place_and_other_scale():
    Q, K, V, O, routed, alpha = _inputs(2, 384, 2, 940, 0.25, out_dtype="f32")
    got = _run(Q, K, V, O, routed, alpha, 2, 64, 40, scale=0.3, out_dtype="f32", inplace=True)
    assert got.element_size() == 4
    assert_close(host_f64(got), _oracle(Q, K, V, O, routed, alpha, 2, 64, 40, 0.3), TOL_BF16,
                 "fp32 in place")


def test_empty_cache_copies_the_ttt_output_bit_for_bit():
    Q, K, V, O, routed, alpha = _inputs(2, 256, 2, 950, 0.3)
    got = host_bits(_run(Q, K, V, O, np.zeros_like(routed), alpha, 2, 64, 16))
    np.testing.assert_array_equal(got, O)
    got = host_bits(_run(Q, K, V, O, routed, alpha, 2, 64, 16))
    np.testing.assert_array_equal(got[:, :64], O[:, :64])  # the first chunk's cache is empty


def test_zero_gate_and_later_chunks_leave_outputs_bitwise_unchanged():
    Q, K, V, O, routed, alpha = _inputs(1, 512, 2, 960, 0.3)
    ref = host_bits(_run(Q, K, V, O, routed, alpha, 2, 128, 32))
    np.testing.assert_array_equal(
        host_bits(_run(Q, K, V, O, routed, np.full_like(alpha, -1.0), 2, 128, 32)), O)
    for c in (0, 1, 2):
        K1, V1, r1 = K.copy(), V.copy(), routed.copy()
        K1[:, (c + 1) * 128:] ^= np.uint16(0x0100)
        V1[:, (c + 1) * 128:] ^= np.uint16(0x0100)
        r1[:, (c + 1) * 128:] = 1 - r1[:, (c + 1) * 128:]
        got = host_bits(_run(Q, K1, V1, O, r1, alpha, 2, 128, 32))
        np.testing.assert_array_equal(got[:, :(c + 2) * 128], ref[:, :(c + 2) * 128])


def test_sr_workload_end_to_end():
    """B=4, T=2048, 16 heads x 64, chunk 64, capacity 256: TTT-Linear output and losses, routing,
    then the readout; sampled rows against the oracle fed the same TTT output and mask."""
    import torch
    print("case: readout SR workload (TTT-Linear -> route -> readout)", flush=True)
    inp = gen.route_inputs(B=4, T=2048, d_model=1024, H=16, dh=64, seed_base=50)
    Q, K, V = dev(inp.Q, "bf16"), dev(inp.K, "bf16"), dev(inp.V, "bf16")
    O, _, loss = ttt.linear_minibatch(Q, K, V, 64, 0.01)
    r = ttt.surprisal_route(loss, K, V, 64, want_kv=False)
    B, T, HD = 4, 2048, 1024
    alpha = gen.normal(970, (HD,), 0.5).astype(np.float32) + np.float32(0.5)
    Q3, K3, V3, O3 = (t.reshape(B, T, HD) for t in (Q, K, V, O))
    out = ttt.cache_readout(Q3, K3, V3, r["mask"], O3, dev(alpha, "f32"), 16, 64, 256)
    torch.cuda.synchronize()
    mask = host_bits(r["mask"])
    print(f"  routed per sequence: {mask.sum(axis=1).tolist()}", flush=True)
    rows = [(b, t) for b in range(4) for t in (0, 63, 64, 700, 1300, 2047)]
    Qh, Kh, Vh = (gen.bf16_bits_to_f32(x.reshape(B, T, HD)) for x in (inp.Q, inp.K, inp.V))
    Oh = host_f64(O3)
    ref = orr.cache_readout_rows(Qh, Kh, Vh, mask, Oh, alpha, 16, 64, 256, 0.125, rows)
    got = np.stack([host_f64(out[b, t]) for b, t in rows])
    assert_close(got, ref, TOL_BF16, "sampled fused rows")
    att_ref = ref - np.stack([Oh[b, t] for b, t in rows])
    att_got = got - np.stack([Oh[b, t] for b, t in rows])
    assert_close(att_got, att_ref, TOL_BF16, "sampled attention contribution")
