"""Expected contents of the bounded cache for a given history.

TEST INFRASTRUCTURE ONLY (see the package docstring).

After n tokens of a sequence with pinned prefix length P and window W, the
logical cache is pinned_view(P, W, [0..n)): the prefix positions, then the
window oldest first ([PS] 03; [KV-Lean] 2.3). Entry i of the window holds
position base + i with base = max(P, n - W) ([KV-Lean] 2.4, 3.2).

Stored bytes: V is stored exactly as given. K is stored rotated at its
absolute position and rounded once to the storage dtype ([PS] 05: keys are
rotated once and reused; the single rounding is the reading taken here, see `rne`).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import rne, rope, spec


def expected_positions(P: int, W: int, n: int) -> np.ndarray:
    """Absolute positions held by the cache after n tokens, prefix then window oldest first."""
    return np.asarray(spec.pinned_view(P, W, range(n)), dtype=np.int64)


def stored_key_bits(k: np.ndarray, pos: np.ndarray, base: float, dtype: str) -> np.ndarray:
    """Bit patterns of the stored keys: RNE_dtype(rotate_float64(k, pos)).

    k: [n, H_kv, D] input values (float64-exact), pos: [n] absolute positions.
    Returns uint16 (bf16) or uint32 (f32) bit patterns of shape [n, H_kv, D].
    """
    k = np.asarray(k, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    kr = rope.rotate(k, np.broadcast_to(pos[:, None], k.shape[:2]), base)
    if dtype == "bf16":
        return rne.f64_to_bf16_bits(kr)
    if dtype == "f32":
        return rne.f64_to_f32(kr).view(np.uint32)
    raise ValueError(dtype)


def expected_view(P: int, W: int, n: int, hist, base: float, dtype: str
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(positions, stored K bits, V values) of the logical cache after n tokens.

    hist(positions) -> (k, v) float64 input values, as in `attn`.
    """
    pos = expected_positions(P, W, n)
    k, v = hist(pos)
    return pos, stored_key_bits(k, pos, base, dtype), np.asarray(v, dtype=np.float64)
