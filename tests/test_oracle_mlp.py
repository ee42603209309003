"""Pins of the gated-MLP oracle (oracle/mlp.py) against facts the mathematics fixes."""
import numpy as np

import gen
import oracle.mlp as om


def test_silu_closed_form_values():
    # SiLU(0) = 0; SiLU(x) = x * sigmoid(x); large positive x -> x, large negative -> 0
    x = np.array([0.0, 1.0, -1.0, 20.0, -20.0])
    sig = np.array([0.5, 1 / (1 + np.e ** -1), 1 / (1 + np.e), 1 / (1 + np.e ** -20),
                    1 / (1 + np.e ** 20)])
    np.testing.assert_allclose(om.silu(x), x * sig, rtol=1e-12, atol=0)
    assert om.silu(np.array([0.0]))[0] == 0.0
    assert abs(om.silu(np.array([40.0]))[0] - 40.0) < 1e-12      # -> x
    assert abs(om.silu(np.array([-40.0]))[0]) < 1e-15             # -> 0
    xs = np.linspace(-6, 6, 25)
    np.testing.assert_allclose(om.silu(-xs), om.silu(xs) - xs, rtol=0, atol=1e-14)  # s(-x) = s(x) - x


def test_single_element_product():
    # d_model = d_ff = 1: z = silu(x g) * (x u)
    z = om.gated_z([[2.0]], [[0.5]], [[3.0]])
    assert abs(z[0, 0] - (1.0 / (1 + np.exp(-1.0))) * 6.0) < 1e-12


def test_gate_zero_or_up_zero_gives_zero():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((5, 4))
    W = rng.standard_normal((4, 3))
    assert not om.gated_z(X, np.zeros((4, 3)), W).any()   # SiLU(0) = 0
    assert not om.gated_z(X, W, np.zeros((4, 3))).any()


def test_linear_in_the_up_path_and_rows_independent():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((6, 5))
    Wg, Wu = rng.standard_normal((5, 4)), rng.standard_normal((5, 4))
    np.testing.assert_allclose(om.gated_z(X, Wg, 3 * Wu), 3 * om.gated_z(X, Wg, Wu), rtol=1e-12)
    np.testing.assert_allclose(om.gated_z_rows(X, Wg, Wu, [4, 1]),
                               om.gated_z(X, Wg, Wu)[[4, 1]], rtol=1e-12)


def test_matches_the_independent_generator_recipe():
    # gen.inplace_mlp builds Z for the scan's inputs in fp32 with its own code
    T, d, dff, C = 64, 32, 48, 32
    inp = gen.inplace_mlp(T, d, dff, C, eta=1e-3, seed_base=610)
    s = 610
    X = gen.normal(s + 1, (T, d))
    Wg = gen.normal(s + 2, (d, dff), 1.0 / np.sqrt(d))
    Wu = gen.normal(s + 3, (d, dff), 1.0 / np.sqrt(d))
    ref = om.gated_z(X, Wg, Wu)
    got = gen.bf16_bits_to_f32(inp.Z[0]).astype(np.float64)
    assert np.abs(got - ref).max() / np.abs(ref).max() < 1e-2
