"""Pins for the oracle's RoPE (CPU only).

RoPE is not defined on the pages beyond naming a decoupled position branch; the
reading is RoFormer's rotation of consecutive pairs.  These tests pin it to
properties of that definition: it is a rotation (norm kept), scores depend only
on the position difference, position 0 is the identity, and it equals the
complex-number form z_i * exp(i * pos * theta_i) with theta_i = base^(-2i/d).
"""
import numpy as np
import pytest

from oracle import rope


@pytest.mark.parametrize("d", [16, 64])
def test_rope_is_norm_preserving(d):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((50, d))
    pos = rng.integers(0, 200000, 50)
    y = rope(x, pos, 10000.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("d", [16, 64])
def test_rope_relative_position(d):
    rng = np.random.default_rng(1)
    q = rng.standard_normal(d)
    k = rng.standard_normal(d)
    for m, n in [(5, 2), (1000, 997), (131071, 131068)]:
        a = rope(q, m, 10000.0) @ rope(k, n, 10000.0)
        b = rope(q, m - n, 10000.0) @ rope(k, 0, 10000.0)
        assert abs(a - b) <= 1e-9 * (1 + abs(b))
    # ...and it does depend on the difference
    assert abs(rope(q, 3, 1e4) @ k - rope(q, 4, 1e4) @ k) > 1e-6


def test_rope_position_zero_is_identity():
    x = np.random.default_rng(2).standard_normal((3, 64))
    assert np.array_equal(rope(x, 0, 10000.0), x)


@pytest.mark.parametrize("d,base", [(16, 10000.0), (64, 10000.0), (64, 500.0)])
def test_rope_matches_complex_rotation(d, base):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, d))
    pos = rng.integers(0, 140000, 20)
    z = x[:, 0::2] + 1j * x[:, 1::2]
    theta = np.exp(-(2.0 * np.arange(d // 2) / d) * np.log(base))
    w = z * np.exp(1j * pos[:, None] * theta[None, :])
    y = rope(x, pos, base)
    assert np.allclose(y[:, 0::2], w.real, atol=1e-9)
    assert np.allclose(y[:, 1::2], w.imag, atol=1e-9)


def test_rope_first_pair_turns_one_radian_per_position():
    # theta_0 = base^0 = 1: pair 0 of e_0 at position p is (cos p, sin p)
    e0 = np.zeros(64)
    e0[0] = 1.0
    y = rope(e0, 2, 10000.0)
    assert np.allclose(y[:2], [np.cos(2.0), np.sin(2.0)], atol=1e-15)
    assert np.all(y[2:] == 0)
