"""Planted mistakes: ring-buffer models with the bugs of [KV-Lean] 1.2 must fail the
checks the GPU cache is held to (logical view == pinned_view, positions base + i).

These models live only here, on the CPU; they show that the checks catch each bug
class, and in particular that some are caught only at or after the first eviction
([KV-Lean] 1.3), which is why the GPU cache tests walk every step up to 3W + P."""
import pytest

from oracle import spec
from oracle.spec import Cell


class OffByOneShift(spec.RingCache):
    """Window read one slot too far: the logical head is shifted by one."""

    def view(self):
        nw = self.count_window()
        head = (spec.window_base(self.P, self.W, self.n) - self.P + 1) % self.W
        return list(self.prefix) + spec.ring_to_list(self.ring, head, nw)


class WrongBaseWhileFilling(spec.RingCache):
    """The 1-based base m - W + 1 of the window (m = tokens after the prefix) computed with
    truncated subtraction ([KV-Lean] 5.2): right once full, wrong (0 instead of 1) before."""

    def view(self):
        nw = self.count_window()
        m = self.n - self.P
        base_1based = max(0, m - self.W + 1)
        head = (base_1based - 1) % self.W
        return list(self.prefix) + spec.ring_to_list(self.ring, head, nw)


class WrongRollingPosition(spec.RingCache):
    """The position recorded with a token is its slot index plus P (reset after each wrap),
    i.e. the absolute position is lost once the ring wraps."""

    def push(self, kv):
        if self.n < self.P:
            self.prefix.append(kv)
        else:
            slot = (self.n - self.P) % self.W
            self.ring[slot] = Cell(self.P + slot, kv.key, kv.val)
        self.n += 1


class HeadTailOrderSwapped(spec.RingCache):
    """Explicit head/tail pointers, with the tail advanced before the write."""

    def __init__(self, P, W):
        super().__init__(P, W)
        self.tail = 0
        self.head = 0
        self.count = 0

    def push(self, kv):
        if self.n < self.P:
            self.prefix.append(kv)
        else:
            self.tail = (self.tail + 1) % self.W      # bug: advance first
            self.ring[self.tail] = kv
            if self.count == self.W:
                self.head = (self.head + 1) % self.W
            else:
                self.count += 1
        self.n += 1

    def view(self):
        return list(self.prefix) + spec.ring_to_list(self.ring, self.head, self.count)


def first_failure(model_cls, P, W):
    """First n at which the model's view differs from the list model (None if never up to 3W+P+3)."""
    r = model_cls(P, W)
    hist = []
    for p in range(3 * W + P + 4):
        cell = Cell(p)
        r.push(cell)
        hist.append(cell)
        view = r.view()
        ok = view == spec.pinned_view(P, W, hist)
        win = view[min(len(hist), P):]
        ok = ok and all(isinstance(c, Cell) for c in win) and spec.position_invariant(win)
        if not ok:
            return len(hist)
    return None


@pytest.mark.parametrize("model", [OffByOneShift, WrongBaseWhileFilling, WrongRollingPosition,
                                   HeadTailOrderSwapped])
def test_each_bug_is_caught(model):
    for P in range(0, 4):
        for W in range(2, 7):
            assert first_failure(model, P, W) is not None, (model.__name__, P, W)


def test_some_bugs_hide_until_the_window_fills():
    # The wrong-position bug is invisible until the ring wraps: it first fails at the first
    # replacement after the window is full (n = P + W + 1).
    for P in range(0, 4):
        for W in range(2, 7):
            assert first_failure(WrongRollingPosition, P, W) == P + W + 1


def test_correct_model_passes():
    for P in range(0, 4):
        for W in range(1, 7):
            assert first_failure(spec.RingCache, P, W) is None
