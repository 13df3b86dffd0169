"""Pins of spec.WindowModel (per-step window length, promotion) and attn.attend_list."""
import numpy as np

from oracle import attn, spec
from oracle.spec import Cell


def test_constant_window_is_pinned_view():
    for P in range(0, 4):
        for W in range(1, 6):
            m = spec.WindowModel(P, W)
            hist = []
            for p in range(3 * W + P + 3):
                m.push(Cell(p))
                hist.append(Cell(p))
                assert m.view() == spec.pinned_view(P, W, hist)


def test_window_change_by_brute_force():
    # After a shrink, the window is the newest w entries; after a growth it refills only
    # with new tokens. Brute force: the window equals the positions > every past frontier.
    rng = np.random.default_rng(0)
    for trial in range(200):
        P = int(rng.integers(0, 4))
        w = int(rng.integers(1, 7))
        m = spec.WindowModel(P, w)
        frontier = P
        n = 0
        for _ in range(40):
            if rng.random() < 0.2:
                w = int(rng.integers(1, 7))
                m.set_window(w)
                frontier = max(frontier, n - w)
            else:
                m.push(Cell(n))
                n += 1
                frontier = max(frontier, n - w)
            want = list(range(min(n, P))) + list(range(max(frontier, P), n))
            assert [c.pos for c in m.view()] == want
            assert len(m.window) <= w


def test_promotion_moves_oldest_window_entries():
    m = spec.WindowModel(2, 4)
    for p in range(10):
        m.push(Cell(p))
    assert [c.pos for c in m.view()] == [0, 1, 6, 7, 8, 9]
    m.promote(2)
    assert [c.pos for c in m.pinned] == [0, 1, 6, 7]
    assert [c.pos for c in m.window] == [8, 9]
    for p in range(10, 16):
        m.push(Cell(p))
    assert [c.pos for c in m.view()] == [0, 1, 6, 7, 12, 13, 14, 15]


def test_attend_list_equals_mask_form_for_the_closed_form_set():
    rng = np.random.default_rng(1)
    k = rng.standard_normal((80, 2, 16))
    v = rng.standard_normal((80, 2, 16))
    h = attn.array_history(k, v)
    for p in (5, 30, 79):
        q = rng.standard_normal((4, 16))
        pos = spec.pinned_view(3, 20, range(p + 1))
        a = attn.attend_list(q, p, h, pos, 2, 10000.0, 0.25)
        b = attn.decode_query(q, p, h, 3, 20, 2, 10000.0, 0.25)
        np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)
