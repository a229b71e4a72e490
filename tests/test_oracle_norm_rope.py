"""Pins of the oracle's RMSNorm + RoPE step (upstream of the MLA cache write): closed
forms, invariances and the rotation as complex multiplication (numpy's complex product, a
library primitive the oracle does not use)."""
import numpy as np

from oracle import oracle


def _rand(T, Dn, Dr, seed=0):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((T, Dn + Dr))
    gamma = rng.standard_normal(Dn)
    ang = rng.uniform(-np.pi, np.pi, (T, Dr // 2))
    return kv, gamma, np.cos(ang), np.sin(ang), ang


def test_rope_is_complex_multiplication():
    kv, gamma, c, s, ang = _rand(5, 16, 64)
    _, rope = oracle.rmsnorm_rope(kv, gamma, c, s, 16, 1e-6)
    z = kv[:, 16:48] + 1j * kv[:, 48:]
    w = z * np.exp(1j * ang)
    np.testing.assert_allclose(rope[:, :32], w.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(rope[:, 32:], w.imag, rtol=0, atol=1e-13)


def test_rope_at_angle_zero_is_identity_and_keeps_pair_norms():
    kv, gamma, c, s, _ = _rand(3, 8, 16, seed=1)
    _, rope0 = oracle.rmsnorm_rope(kv, gamma, np.ones_like(c), np.zeros_like(s), 8, 1e-6)
    assert np.array_equal(rope0, kv[:, 8:])
    _, rope = oracle.rmsnorm_rope(kv, gamma, c, s, 8, 1e-6)
    n_in = kv[:, 8:16] ** 2 + kv[:, 16:] ** 2
    n_out = rope[:, :8] ** 2 + rope[:, 8:] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-13)


def test_rmsnorm_closed_forms():
    T, Dn = 4, 32
    x = np.zeros((T, Dn + 2))
    x[:, :Dn] = np.array([3.0, -3.0, 0.5, 7.0])[:, None]        # constant rows
    g = np.linspace(-2, 2, Dn)
    nope, _ = oracle.rmsnorm_rope(x, g, np.ones((T, 1)), np.zeros((T, 1)), Dn, 0.0)
    # a constant row c normalises to sign(c)
    np.testing.assert_allclose(nope, np.sign(x[:, :1]) * g[None, :], rtol=0, atol=1e-15)
    # eps: a row of ones with eps = 3 normalises to 1 / 2
    ones = np.ones((1, Dn + 2))
    nope, _ = oracle.rmsnorm_rope(ones, np.ones(Dn), np.ones((1, 1)), np.zeros((1, 1)), Dn, 3.0)
    np.testing.assert_allclose(nope, 0.5, rtol=0, atol=1e-15)


def test_rmsnorm_unit_rms_and_scale_invariance():
    kv, _, c, s, _ = _rand(6, 512, 64, seed=2)
    nope, _ = oracle.rmsnorm_rope(kv, np.ones(512), c, s, 512, 0.0)
    np.testing.assert_allclose((nope ** 2).mean(axis=1), 1.0, rtol=1e-13)
    nope2, _ = oracle.rmsnorm_rope(kv * 37.5, np.ones(512), c, s, 512, 0.0)
    np.testing.assert_allclose(nope2, nope, rtol=1e-13, atol=0)


def test_bf16_inputs_widen_exactly():
    # bf16 bit patterns: 1.0 = 0x3F80, -2.0 = 0xC000, 0.5 = 0x3F00
    u = np.array([[0x3F80, 0xC000, 0x3F00, 0x3F80]], np.uint16)
    assert np.array_equal(oracle.widen(u), [[1.0, -2.0, 0.5, 1.0]])
