"""Rotary position encoding at absolute positions, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[PS] 05: positions keep counting up after eviction ("Continue PE"), so a key
is rotated once, at the absolute position of its token, and reused as is for
as long as it stays in the cache.

The pages do not fix a rotary convention or base. The reading taken here is
the rotate-half pairing: element i is paired with element i + D/2, and the
pair is turned by the angle p * theta_i with theta_i = base ** (-2 i / D),
base 10000, rounded once to the nearest float64 (the correctly rounded power:
a power routine that is only faithful can land one ulp off, which moves the
angle of a late position by p ulps of theta). The angle is the float64 product
of p and theta_i; cos and sin are float64; the rotated pair is
(x c - y s, x s + y c), each product and sum rounded separately (no fused
multiply-add).
"""
from __future__ import annotations

import functools
from fractions import Fraction

import mpmath
import numpy as np


def inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base ** (-2 i / D) for i in [0, D/2), rounded once to float64.

    The power is evaluated at 300 bits (mpmath) with the exact rational exponent and
    then rounded to the nearest double, so theta_i is the float64 nearest to the real
    value, whatever the platform's power routine does."""
    return _inv_freq(int(head_dim), float(base)).copy()


@functools.lru_cache(maxsize=None)
def _inv_freq(head_dim: int, base: float) -> np.ndarray:
    out = np.empty(head_dim // 2, dtype=np.float64)
    with mpmath.workprec(300):
        b = mpmath.mpf(float(base))
        for i in range(head_dim // 2):
            e = Fraction(-2 * i, head_dim)
            man, exp = mpmath.power(b, mpmath.mpf(e.numerator) / e.denominator).man_exp
            # the 300-bit value as an exact fraction; int / int division rounds to nearest
            out[i] = float(Fraction(int(man)) * Fraction(2) ** int(exp))
    return out


def angles(pos, head_dim: int, base: float) -> np.ndarray:
    """phi[..., i] = p * theta_i in float64 for positions `pos` (any shape)."""
    pos = np.asarray(pos, dtype=np.float64)
    return pos[..., None] * inv_freq(head_dim, base)


def rotate(x, pos, base: float) -> np.ndarray:
    """Rotate vectors x[..., D] at positions pos[...] (broadcast to x's leading dims)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    phi = angles(np.broadcast_to(np.asarray(pos), x.shape[:-1]), D, base)
    c = np.cos(phi)
    s = np.sin(phi)
    a = x[..., :h]
    b = x[..., h:]
    out = np.empty_like(x)
    out[..., :h] = a * c - b * s
    out[..., h:] = a * s + b * c
    return out
