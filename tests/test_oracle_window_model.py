"""Pins of spec.WindowModel (per-step window length, promotion) and attn.attend_list."""
import numpy as np

from oracle import attn, rope, spec
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


def test_attend_view_equals_mask_form_for_the_closed_form_set():
    # Both PE modes: on the closed-form set the list form must match the mask form
    # (continue) and reset_positions (reset), including queries inside the prefix.
    rng = np.random.default_rng(1)
    k = rng.standard_normal((80, 2, 16))
    v = rng.standard_normal((80, 2, 16))
    h = attn.array_history(k, v)
    for pe in ("continue", "reset"):
        for p in (1, 5, 30, 79):
            q = rng.standard_normal((4, 16))
            pos = spec.pinned_view(3, 20, range(p + 1))
            a = attn.attend_view(q, p, h, pos, 2, 10000.0, 0.25, pe)
            b = attn.decode_query(q, p, h, 3, 20, 2, 10000.0, 0.25, pe)
            np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
            np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_attend_view_shrunk_window_is_a_smaller_window():
    # A window shrunk to w at once and then filled again equals the constant window w
    # once w new tokens have arrived (every older entry has left either way).
    rng = np.random.default_rng(2)
    k = rng.standard_normal((120, 2, 16))
    v = rng.standard_normal((120, 2, 16))
    h = attn.array_history(k, v)
    m = spec.WindowModel(4, 40)
    for p in range(60):
        m.push(p)
    m.set_window(9)
    for p in range(60, 100):
        m.push(p)
        if p >= 69:
            q = rng.standard_normal((4, 16))
            a = attn.attend_view(q, p, h, m.view(), 2, 10000.0, 0.25)
            b = attn.decode_query(q, p, h, 4, 9, 2, 10000.0, 0.25)
            np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)


def test_promoted_tokens_stay_visible():
    # After promotion the promoted positions are attended forever: the output equals the
    # mask form with those positions forced visible (a hand-built logit mask).
    rng = np.random.default_rng(3)
    k = rng.standard_normal((90, 1, 8))
    v = rng.standard_normal((90, 1, 8))
    h = attn.array_history(k, v)
    m = spec.WindowModel(2, 6)
    for p in range(20):
        m.push(p)
    m.promote(3)                      # positions 14, 15, 16
    for p in range(20, 90):
        m.push(p)
    q = rng.standard_normal((1, 8))
    out, lse = attn.attend_view(q, 89, h, m.view(), 1, 10000.0, 1.0)
    keep = [0, 1, 14, 15, 16] + list(range(84, 90))
    qr = rope.rotate(q, np.full(1, 89), 10000.0)[0]
    kr = rope.rotate(k[keep], np.asarray(keep)[:, None], 10000.0)[:, 0]
    s = kr @ qr
    w = np.exp(s - s.max())
    np.testing.assert_allclose(out[0], (w / w.sum()) @ v[keep, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], s.max() + np.log(w.sum()), rtol=0, atol=1e-12)
