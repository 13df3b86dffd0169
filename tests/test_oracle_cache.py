"""Pins of oracle.cache: expected positions equal the physical ring model read back, and the
stored key of position 0 is the input key itself (rotation by angle 0, exact in bf16/f32)."""
import numpy as np
import torch

from oracle import cache, rne, spec
from oracle.spec import Cell


def test_expected_positions_match_ring_model():
    for P in range(0, 4):
        for W in range(1, 6):
            r = spec.RingCache(P, W)
            for p in range(3 * W + P + 3):
                r.push(Cell(p))
                assert [c.pos for c in r.view()] == cache.expected_positions(P, W, p + 1).tolist()


def test_position_zero_key_is_stored_unchanged():
    k16 = torch.randn(1, 4, 128).to(torch.bfloat16)
    bits = cache.stored_key_bits(k16.double().numpy(), np.array([0]), 10000.0, "bf16")
    np.testing.assert_array_equal(bits, k16.view(torch.int16).numpy().view(np.uint16))
    k32 = torch.randn(1, 4, 64)
    bits32 = cache.stored_key_bits(k32.double().numpy(), np.array([0]), 10000.0, "f32")
    np.testing.assert_array_equal(bits32, k32.numpy().view(np.uint32))


def test_stored_key_is_rounded_rotation():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((5, 2, 64))
    pos = np.array([7, 100, 5000, 65536, 131071])
    bits = cache.stored_key_bits(k, pos, 10000.0, "bf16")
    vals = rne.bf16_bits_to_f64(bits)
    from oracle import rope
    exact = rope.rotate(k, np.broadcast_to(pos[:, None], (5, 2)), 10000.0)
    # one rounding: within half a bfloat16 ulp of the float64 rotation
    ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    assert np.all(np.abs(vals - exact) <= ulp / 2)
