"""Pins of oracle.rne: exact rational rounding, the library's float32 -> bfloat16 cast,
IEEE special values and the double-rounding case that separates one rounding from two."""
import math
import struct
from fractions import Fraction

import numpy as np
import torch

from oracle import rne


def exact_bf16(x: float) -> float:
    """Round a float64 to bfloat16 with exact rational arithmetic (ties to even)."""
    if math.isnan(x):
        return math.nan
    if math.isinf(x) or x == 0.0:
        return x
    sign = -1.0 if x < 0 else 1.0
    a = Fraction(abs(x))
    m, e = math.frexp(abs(x))              # abs(x) = m * 2**e, m in [0.5, 1)
    E = e - 1                              # abs(x) in [2**E, 2**(E+1))
    quantum = Fraction(2) ** (E - 7) if E >= -126 else Fraction(2) ** -133
    q = a / quantum
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(r)


def bits_of_bf16_value(v: float) -> int:
    if math.isnan(v):
        return 0x7FC0
    return struct.unpack("<I", struct.pack("<f", v))[0] >> 16 if v == v else 0


def test_matches_exact_rational_rounding():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(20000),
        rng.standard_normal(5000) * 1e30,
        rng.standard_normal(5000) * 1e-38,      # around the bfloat16 subnormal range
        rng.standard_normal(2000) * 1e-40,
        rng.standard_normal(2000) * 3e38,       # overflow region
        np.ldexp(rng.integers(1 << 52, 1 << 53, 4000).astype(np.float64), -52),  # [1, 2)
    ])
    got = rne.f64_to_bf16_bits(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        want = exact_bf16(x)
        wb = struct.unpack("<I", struct.pack("<f", want))[0] >> 16
        assert g == wb, (x, hex(g), hex(wb))


def test_ties_go_to_even():
    one = 1.0
    ulp = 2.0 ** -7
    cases = {
        one + ulp / 2: 1.0,                     # tie, 1.0 is even
        one + 3 * ulp / 2: one + 2 * ulp,       # tie, rounds up to the even neighbour
        one + ulp / 2 + 2.0 ** -40: one + ulp,  # just above the tie
        -(one + ulp / 2): -1.0,
    }
    for x, want in cases.items():
        assert rne.bf16_bits_to_f64(rne.f64_to_bf16_bits(np.array([x])))[0] == want


def test_single_rounding_differs_from_double():
    # 1 + 2**-8 + 2**-40: one rounding goes up to 1 + 2**-7; rounding to float32 first lands
    # exactly on the tie 1 + 2**-8, which then goes to the even 1.0.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert rne.round_to(np.array([x]), "bf16")[0] == 1.0 + 2.0 ** -7
    twice = torch.tensor([x], dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
    assert twice.double().item() == 1.0


def test_agrees_with_torch_on_float32_inputs():
    # For inputs already representable in float32 the library cast float32 -> bfloat16 (RNE) is a
    # single rounding, so it must agree bit for bit.
    rng = np.random.default_rng(1)
    x32 = (rng.standard_normal(200000) * np.exp(rng.uniform(-80, 80, 200000))).astype(np.float32)
    x32 = np.concatenate([x32, np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38,
                                         1.1754944e-38, 9.2e-41, -9.2e-41], dtype=np.float32)])
    ours = rne.f64_to_bf16_bits(x32.astype(np.float64))
    theirs = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, theirs)


def test_special_values():
    x = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e300, -1e300, 5e-324])
    b = rne.f64_to_bf16_bits(x)
    assert b[0] == 0x0000 and b[1] == 0x8000
    assert b[2] == 0x7F80 and b[3] == 0xFF80
    assert b[4] & 0x7FFF == 0x7FC0
    assert b[5] == 0x7F80 and b[6] == 0xFF80
    assert b[7] == 0x0000


def test_f32_is_single_rne():
    rng = np.random.default_rng(2)
    xs = rng.standard_normal(5000) * np.exp(rng.uniform(-60, 60, 5000))
    got = rne.f64_to_f32(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        a = Fraction(x)
        m, e = math.frexp(abs(x))
        E = e - 1
        quantum = Fraction(2) ** (E - 23) if E >= -126 else Fraction(2) ** -149
        q = abs(a) / quantum
        n = q.numerator // q.denominator
        rem = q - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        want = math.copysign(float(n * quantum), x)
        assert g == want
