"""The generators' bf16 packing against torch's own fp32 -> bf16 conversion, and seed determinism."""
import numpy as np
import torch

import gen


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32) * 10.0,
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, np.inf, -np.inf], np.float32),
        # exact ties: low 16 bits == 0x8000, both parities of the kept mantissa
        np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000], np.uint32).view(np.float32),
    ])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    np.testing.assert_array_equal(gen.bf16_bits_to_f32(ours),
                                  torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_nan_stays_nan():
    x = np.array([np.nan], np.float32)
    assert np.isnan(gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x)))[0]


def test_generators_are_seeded():
    a = gen.inplace_mlp(128, 64, 96, 32, seed_base=90)
    b = gen.inplace_mlp(128, 64, 96, 32, seed_base=90)
    np.testing.assert_array_equal(a.Z, b.Z)
    np.testing.assert_array_equal(a.V, b.V)
    np.testing.assert_array_equal(a.W0, b.W0)
    r = gen.route_inputs(B=2, T=256, d_model=64, H=2, dh=16)
    assert r.meta["outliers"].shape == (2, round(0.02 * 256))
