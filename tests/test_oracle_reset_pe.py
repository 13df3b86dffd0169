"""Pins of the Reset PE reference ([PS] 05): the literal renumbering of the cache list,
equality with Continue PE wherever nothing was renumbered or no prefix exists, and that
it does differ once the window has slid past a prefix."""
import numpy as np

from oracle import attn, rope, spec


def literal_reset(q, p, k, v, P, W, scale):
    """Rotate every cached token at its index in the list [prefix, window] and the query at
    the index of the newest entry; softmax by hand."""
    cache = spec.pinned_view(P, W, range(p + 1))
    idx = np.arange(len(cache))
    qr = rope.rotate(q[None], np.array([idx[-1]]), 10000.0)[0]
    kr = rope.rotate(k[cache], idx, 10000.0)
    s = kr @ qr * scale
    e = np.exp(s - s.max())
    return (e[:, None] * v[cache]).sum(0) / e.sum()


def test_matches_literal_renumbering():
    rng = np.random.default_rng(0)
    D = 16
    for P, W in [(3, 5), (0, 4), (6, 2), (1, 1)]:
        n = 3 * W + P + 4
        k = rng.standard_normal((n, 1, D))
        v = rng.standard_normal((n, 1, D))
        h = attn.array_history(k, v)
        for p in range(n):
            q = rng.standard_normal((1, D))
            out, _ = attn.decode_query(q, p, h, P, W, 1, 10000.0, 0.3, pe="reset")
            ref = literal_reset(q[0], p, k[:, 0], v[:, 0], P, W, 0.3)
            np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


def test_equals_continue_before_the_window_slides_and_without_prefix():
    rng = np.random.default_rng(1)
    D = 16
    for P, W in [(4, 6), (0, 5)]:
        n = 4 * W + P
        k = rng.standard_normal((n, 2, D))
        v = rng.standard_normal((n, 2, D))
        h = attn.array_history(k, v)
        for p in range(n):
            q = rng.standard_normal((4, D))
            a = attn.decode_query(q, p, h, P, W, 2, 10000.0, 0.25)
            b = attn.decode_query(q, p, h, P, W, 2, 10000.0, 0.25, pe="reset")
            if p + 1 <= P + W or P == 0:
                np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-9)


def test_differs_after_the_window_slides():
    rng = np.random.default_rng(2)
    P, W, D = 4, 6, 32
    n = 60
    k = rng.standard_normal((n, 1, D))
    v = rng.standard_normal((n, 1, D))
    q = rng.standard_normal((1, D))
    h = attn.array_history(k, v)
    a = attn.decode_query(q, n - 1, h, P, W, 1, 10000.0, 0.25)[0]
    b = attn.decode_query(q, n - 1, h, P, W, 1, 10000.0, 0.25, pe="reset")[0]
    assert np.abs(a - b).max() > 1e-3


def test_reset_positions_closed_form():
    q, kp = attn.reset_positions(10, 4, 30, np.array([0, 9, 27, 28, 29, 30]))
    assert q == 13                                   # base = 27 -> 10 + 3
    assert kp.tolist() == [0, 9, 10, 11, 12, 13]
    q, kp = attn.reset_positions(10, 4, 7, np.array([0, 7]))
    assert q == 7 and kp.tolist() == [0, 7]          # inside the prefix: unchanged
