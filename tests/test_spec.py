"""Pins of the list model (oracle.spec) against the pages' worked example,
closed forms and brute force over small windows."""
import json
import os

import pytest

from oracle import spec
from oracle.spec import Cell


def test_guard_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "kvlean_guard_step.json")))
    assert spec.step(g["w"], g["cache"], g["push"]) == g["expect"]


@pytest.mark.parametrize("w", range(0, 9))
def test_step_identity_brute_force(w):
    # [KV-Lean] 2.4: lastWindow w (xs ++ [kv]) = step w (lastWindow w xs) kv, for every history
    # length up to 3w + 3 (not full, exactly full, first eviction and steady replacement).
    for n in range(0, 3 * w + 4):
        xs = list(range(n))
        kv = n
        assert spec.last_window(w, xs + [kv]) == spec.step(w, spec.last_window(w, xs), kv)


@pytest.mark.parametrize("w", range(0, 9))
def test_run_correct_and_invariants(w):
    # [KV-Lean] 4.2 run_correct, 2.4 length bound, 3.2 position invariant with base = max(0, n - w)
    for n in range(0, 3 * w + 4):
        toks = [Cell(p) for p in range(n)]
        c = spec.run(w, toks)
        assert spec.valid(w, toks, c)
        assert spec.length_ok(w, c)
        assert spec.position_invariant(c)
        if c:
            assert c[0].pos == max(0, n - w) == spec.window_base(0, w, n)


def test_step_preserves_valid_both_cases():
    # [KV-Lean] 4.1: valid before a step implies valid after it, in the not-full and full cases.
    for w in range(1, 7):
        for n in range(0, 3 * w + 2):
            xs = list(range(n))
            c = spec.last_window(w, xs)
            assert spec.valid(w, xs + [n], spec.step(w, c, n))


def test_drop_append_identity_corrected():
    # The page prints (xs ++ [a]).drop(len + 1 - w) = xs.drop(len - w) ++ [a]; its right side has one
    # element too many. The form that holds (and that the step lemma needs) drops len + 1 - w on both
    # sides, for 1 <= w <= len + 1.
    for n in range(0, 12):
        xs = list(range(n))
        a = "a"
        for w in range(1, n + 2):
            lhs = (xs + [a])[n + 1 - w:]
            assert lhs == xs[n + 1 - w:] + [a]
            assert len(lhs) == w
            if w <= n:
                assert lhs == (xs[n - w:] + [a])[1:]
        # the printed form fails whenever w <= n
        for w in range(1, n + 1):
            assert (xs + [a])[n + 1 - w:] != xs[n - w:] + [a]


def test_visible_count_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "ps_visible_count.json")))
    for t in g["t_values"]:
        assert len(spec.visible_1based(g["P"], g["W"], t)) == g["expect_count"]


def test_visible_set_closed_form_small():
    # A(t) = [1,P] u [max(P+1, t-W+1), t] against a direct enumeration of its definition:
    # a 1-based position s is visible iff s <= t and (s <= P or t - s < W).
    for P in range(0, 5):
        for W in range(1, 6):
            for t in range(1, 3 * W + P + 4):
                direct = {s for s in range(1, t + 1) if s <= P or t - s < W}
                assert spec.visible_1based(P, W, t) == direct
                zero_based = {j for j in range(t) if spec.visible(P, W, t - 1, j)}
                assert zero_based == {s - 1 for s in direct}


def test_cache_after_n_tokens_is_visible_set():
    # The cache after n tokens holds exactly A(n) (0-based: positions the query at p = n - 1 sees).
    for P in range(0, 5):
        for W in range(1, 6):
            for n in range(1, 3 * W + P + 4):
                view = spec.pinned_view(P, W, range(n))
                assert view == sorted(s - 1 for s in spec.visible_1based(P, W, n))
                assert len(view) == min(n, P + W)


def test_ring_cache_simulates_list_model():
    # [KV-Lean] 3.4: the ring with a write cursor, read back as a list, equals the list model after
    # every push; [KV-Lean] 1.3: this covers not-full, exactly-full and the first replacement.
    for P in range(0, 5):
        for W in range(1, 7):
            r = spec.RingCache(P, W)
            hist = []
            for p in range(3 * W + P + 4):
                cell = Cell(p)
                r.push(cell)
                hist.append(cell)
                view = r.view()
                assert view == spec.pinned_view(P, W, hist)
                win = view[min(len(hist), P):]
                assert spec.position_invariant(win)
                if win:
                    assert win[0].pos == spec.window_base(P, W, len(hist))


def test_ring_slot_of_position():
    # The window entry at position p >= P lives in ring slot (p - P) mod W; the first window token
    # (p = P) lands in slot 0.
    P, W = 3, 4
    r = spec.RingCache(P, W)
    for p in range(40):
        r.push(Cell(p))
        if p >= P:
            assert r.ring[(p - P) % W].pos == p
