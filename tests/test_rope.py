"""Pins of oracle.rope: the complex-number form of the rotation, norm preservation,
identity at position 0, logits that depend only on the relative offset, and theta_i as the
float64 nearest to base^(-2i/D)."""
import math

import mpmath
import numpy as np

from oracle import rope


def complex_rotate(x, pos, base):
    """Rotation written as complex multiplication: z_i = x_i + 1j * x_{i+D/2}, times e^{1j p theta_i}."""
    D = x.shape[-1]
    h = D // 2
    theta = np.array([math.pow(float(base), (-2.0 * i) / D) for i in range(h)])
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * (np.asarray(pos, dtype=np.float64)[..., None] * theta))
    return np.concatenate([z.real, z.imag], axis=-1)


def test_direction_on_a_unit_vector():
    x = np.zeros((1, 4))
    x[0, 0] = 1.0                                   # pair (0, 2) = (1, 0)
    r = rope.rotate(x, np.array([1]), 10000.0)
    assert np.allclose(r[0], [np.cos(1.0), 0.0, np.sin(1.0), 0.0], atol=0, rtol=1e-15)


def test_matches_complex_form():
    rng = np.random.default_rng(0)
    for D in (64, 128):
        x = rng.standard_normal((300, D))
        pos = rng.integers(0, 200000, 300)
        a = rope.rotate(x, pos, 10000.0)
        b = complex_rotate(x, pos, 10000.0)
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def test_position_zero_is_identity_exactly():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((10, 128))
    np.testing.assert_array_equal(rope.rotate(x, np.zeros(10, dtype=np.int64), 10000.0), x)


def test_pair_norms_preserved():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((100, 128))
    pos = rng.integers(0, 131072, 100)
    r = rope.rotate(x, pos, 10000.0)
    n0 = x[:, :64] ** 2 + x[:, 64:] ** 2
    n1 = r[:, :64] ** 2 + r[:, 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-13)


def test_logits_depend_only_on_offset():
    rng = np.random.default_rng(3)
    q = rng.standard_normal(128)
    k = rng.standard_normal(128)
    for p, j, delta in [(10, 3, 1000), (40000, 35000, 57), (5, 5, 99999)]:
        s0 = rope.rotate(q[None], np.array([p]), 10000.0)[0] @ rope.rotate(k[None], np.array([j]), 10000.0)[0]
        s1 = rope.rotate(q[None], np.array([p + delta]), 10000.0)[0] @ \
            rope.rotate(k[None], np.array([j + delta]), 10000.0)[0]
        assert abs(s0 - s1) < 1e-9 * max(1.0, abs(s0))


def test_inv_freq_closed_form():
    th = rope.inv_freq(128, 10000.0)
    assert th[0] == 1.0
    np.testing.assert_allclose(th[1:] / th[:-1], 10000.0 ** (-2.0 / 128), rtol=1e-14)
    np.testing.assert_allclose(th[-1], 10000.0 ** (-126.0 / 128), rtol=1e-15)


def test_inv_freq_is_the_nearest_double():
    # correct rounding by its definition: the real value lies within half an ulp of theta_i
    # (checked at 600 bits, twice the oracle's working precision)
    for D in (64, 128):
        for base in (10000.0, 500000.0):
            th = rope.inv_freq(D, base)
            with mpmath.workprec(600):
                for i, t in enumerate(th):
                    exact = mpmath.power(mpmath.mpf(base), mpmath.mpf(-2 * i) / D)
                    half = (mpmath.mpf(math.nextafter(t, math.inf)) - mpmath.mpf(t)) / 2
                    assert abs(exact - mpmath.mpf(t)) <= half, (D, base, i)


def test_inv_freq_special_values():
    th = rope.inv_freq(128, 10000.0)
    assert th[32] == 0.01                      # 10000^(-1/2)
    # a faithful power routine can round this one the other way (one ulp below)
    assert th[2] == float.fromhex("0x1.7ff2224115d9ap-1")
    # the platform's correctly rounded pow agrees at every frequency of the tested bases
    for D in (64, 128):
        for base in (10000.0, 500000.0, 1e6):
            th = rope.inv_freq(D, base)
            assert all(math.pow(base, (-2.0 * i) / D) == th[i] for i in range(D // 2))
