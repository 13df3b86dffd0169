"""Single rounding of float64 values to the storage types, to nearest, ties to even.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages never state how a rotated key is rounded for storage. The reading
taken here: the key is rotated in float64 and rounded once to the storage
type (bfloat16 or float32), round to nearest with ties to even. Rounding
float64 -> float32 -> bfloat16 instead would round twice and differs from a
single rounding on a small fraction of inputs.
"""
from __future__ import annotations

import numpy as np

_MAN_BITS = 52
_EXP_MASK = 0x7FF
_MAN_MASK = (1 << 52) - 1


def f64_to_bf16_bits(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float64 values, one rounding to nearest even.

    Works on the float64 bit fields with integer arithmetic:
    * NaN -> the quiet NaN 0x7FC0 with the input's sign; +-inf -> +-inf.
    * Results in the bfloat16 normal range keep 7 fraction bits; a carry out
      of the fraction moves into the exponent, and one out of the largest
      exponent gives infinity.
    * Results below 2**-126 become bfloat16 subnormals (multiples of 2**-133),
      rounded the same way; float64 subnormals round to a signed zero.
    """
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    u = x.view(np.uint64).astype(np.uint64)
    sign = ((u >> np.uint64(63)) << np.uint64(15)).astype(np.uint64)
    e = ((u >> np.uint64(_MAN_BITS)) & np.uint64(_EXP_MASK)).astype(np.int64)
    m = u & np.uint64(_MAN_MASK)
    out = np.zeros(x.shape, dtype=np.uint64)

    is_nan = (e == _EXP_MASK) & (m != 0)
    is_inf = (e == _EXP_MASK) & (m == 0)
    E = e - 1023

    # Normal bfloat16 results: unbiased exponent in [-126, 127] (larger overflows).
    norm = (e != _EXP_MASK) & (e != 0) & (E >= -126)
    if norm.any():
        mm = m[norm]
        kept = mm >> np.uint64(45)
        rem = mm & np.uint64((1 << 45) - 1)
        half = np.uint64(1 << 44)
        body = (np.uint64(0) + (E[norm] + 127).astype(np.uint64)) << np.uint64(7) | kept
        up = (rem > half) | ((rem == half) & ((body & np.uint64(1)) == np.uint64(1)))
        body = body + up.astype(np.uint64)
        body = np.where(body >= np.uint64(0x7F80), np.uint64(0x7F80), body)
        out[norm] = body

    # Subnormal bfloat16 results: value = (2**52 + m) * 2**(E - 52), quantum 2**-133.
    sub = (e != _EXP_MASK) & (e != 0) & (E < -126)
    if sub.any():
        full = m[sub] | np.uint64(1 << 52)
        s = (-E[sub] - 81).astype(np.int64)          # right shift that leaves units of 2**-133
        res = np.zeros(full.shape, dtype=np.uint64)
        ok = s < 64
        ss = s[ok].astype(np.uint64)
        f = full[ok]
        kept = f >> ss
        rem = f & ((np.uint64(1) << ss) - np.uint64(1))
        half = np.uint64(1) << (ss - np.uint64(1))
        up = (rem > half) | ((rem == half) & ((kept & np.uint64(1)) == np.uint64(1)))
        res[ok] = kept + up.astype(np.uint64)
        out[sub] = res

    out[is_inf] = np.uint64(0x7F80)
    out[is_nan] = np.uint64(0x7FC0)
    out = out | sign
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_f32(x) -> np.ndarray:
    """float64 -> float32 with one rounding to nearest even (NumPy's cast is IEEE RNE)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_to(x, dtype: str) -> np.ndarray:
    """Stored value in float64 after rounding once to `dtype` ("bf16" or "f32")."""
    if dtype == "bf16":
        return bf16_bits_to_f64(f64_to_bf16_bits(x))
    if dtype == "f32":
        return f64_to_f32(x).astype(np.float64)
    raise ValueError(dtype)
