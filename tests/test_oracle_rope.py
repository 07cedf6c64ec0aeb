"""Pins of the oracle's partial RoPE: an independent complex-number form,
closed-form values and the rotation invariants."""
import numpy as np

from oracle.rope import apply_rope


def _complex_form(x, p):
    # RoFormer's complex form: pair (x_{2i}, x_{2i+1}) as x_{2i} + i x_{2i+1},
    # multiplied by exp(i p theta_i), theta_i = base^(-2i/d) over the d = 64
    # rotated dims.
    D = x.shape[-1]
    y = x.astype(np.float64).copy()
    z = x[D - 64::2] + 1j * x[D - 64 + 1::2]
    theta = 10000.0 ** (-2.0 * np.arange(32) / 64.0)
    z = z * np.exp(1j * p * theta)
    y[D - 64::2] = z.real
    y[D - 64 + 1::2] = z.imag
    return y


def test_matches_complex_form():
    rng = np.random.default_rng(0)
    for D in (64, 128, 512):
        for p in (0, 1, 7, 4095, 131071, 1048575):
            x = rng.standard_normal(D)
            np.testing.assert_allclose(apply_rope(x, p), _complex_form(x, p), rtol=0, atol=1e-12)


def test_closed_form_values():
    x = np.zeros(128)
    x[64] = 1.0                   # first rotated pair, theta_0 = 1
    y = apply_rope(x, 1)
    assert abs(y[64] - np.cos(1.0)) < 1e-15 and abs(y[65] - np.sin(1.0)) < 1e-15
    x = np.zeros(128)
    x[127] = 1.0                  # last pair's odd element, theta_31 = 10000^(-31/32)
    y = apply_rope(x, 1000)
    a = 1000 * 10000.0 ** (-31 / 32)
    assert abs(y[126] + np.sin(a)) < 1e-13 and abs(y[127] - np.cos(a)) < 1e-13


def test_invariants():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(512)
    k = rng.standard_normal(512)
    assert np.array_equal(apply_rope(q, 0), q)
    y = apply_rope(q, 12345)
    assert np.array_equal(y[:448], q[:448])
    assert abs(np.linalg.norm(y) - np.linalg.norm(q)) < 1e-12
    d1 = apply_rope(q, 1000) @ apply_rope(k, 900)
    d2 = apply_rope(q, 5100) @ apply_rope(k, 5000)
    assert abs(d1 - d2) < 1e-10
    # batched positions equal per-row calls
    X = rng.standard_normal((5, 128))
    P = np.array([0, 3, 99, 1 << 17, 1 << 20])
    Y = apply_rope(X, P)
    for i in range(5):
        np.testing.assert_array_equal(Y[i], apply_rope(X[i], P[i]))
