"""List model of the bounded KV cache and the visible-set predicate.

TEST INFRASTRUCTURE ONLY (see the package docstring).

A cache entry is any Python value; where positions matter an entry is a
``Cell(pos, key, val)``. Lists are oldest first.
"""
from __future__ import annotations

from typing import Any, List, NamedTuple, Sequence


class Cell(NamedTuple):
    """One cached token: absolute 0-based position plus its key and value
    ([KV-Lean] 3.2 models a cell as a position with a key and a value vector)."""
    pos: int
    key: Any = None
    val: Any = None


def last_window(w: int, hs: Sequence) -> list:
    """The last min(w, len(hs)) entries of the history ([KV-Lean] 2.3).

    Drops the first len(hs) - min(w, len(hs)) entries; the subtraction never
    goes below zero because of the min, so no truncated arithmetic is needed
    ([KV-Lean] 4.3, 5.2).
    """
    hs = list(hs)
    keep = min(w, len(hs))
    return hs[len(hs) - keep:]


def valid(w: int, hs: Sequence, c: Sequence) -> bool:
    """A cache state is valid for history hs iff it equals the last window of hs ([KV-Lean] 2.3)."""
    return list(c) == last_window(w, hs)


def step(w: int, c: Sequence, kv) -> list:
    """One generation step of the fixed-length window ([KV-Lean] 2.2, 3.3).

    Append the new entry at the tail; if the list is now longer than w,
    drop the oldest entry. (The branch condition is lost in the page's
    extraction; "longer than W evicts the head" is what 2.2 states and the
    reading used here.)
    """
    c2 = list(c) + [kv]
    if len(c2) > w:
        return c2[1:]
    return c2


def run(w: int, tokens: Sequence) -> list:
    """Fold `step` over the tokens starting from the empty cache ([KV-Lean] 4.2)."""
    c: list = []
    for kv in tokens:
        c = step(w, c, kv)
    return c


def length_ok(w: int, c: Sequence) -> bool:
    """The length invariant: a cache never holds more than w entries ([KV-Lean] 2.4, 3.1)."""
    return len(c) <= w


def position_invariant(c: Sequence[Cell]) -> bool:
    """There is a base such that entry i sits at absolute position base + i ([KV-Lean] 3.2)."""
    if not c:
        return True
    base = c[0].pos
    return all(cell.pos == base + i for i, cell in enumerate(c))


def window_base(P: int, W: int, n: int) -> int:
    """Absolute position of the oldest window entry after n tokens (0-based).

    The window holds positions [max(P, n - W), n). Signed arithmetic with a max,
    not base = n - W + 1 with truncated subtraction, which the Lean article shows
    to be wrong while the window is not yet full ([KV-Lean] 2.4, 5.2).
    """
    return max(P, n - W)


def pinned_view(P: int, W: int, hs: Sequence) -> list:
    """Logical contents of the prefix-pinned cache after history hs.

    The first P entries are never evicted; the rest is a fixed-length window
    of the last W entries ([PS] 03: the prefix KV is computed once and kept,
    the window drops its oldest entry once it holds more than W).
    """
    hs = list(hs)
    return hs[:P] + last_window(W, hs[P:])


def visible_1based(P: int, W: int, t: int) -> set:
    """The set A(t) of 1-based positions the query at position t attends to.

    [PS] 03: the pinned prefix [1, P] together with the recent window
    [max(P + 1, t - W + 1), t]. For a query inside the prefix (t <= P) the
    page states nothing; the reading taken here is plain causal attention,
    A(t) = [1, t], which is also what the union formula gives when the
    prefix part is cut at t.
    """
    if t <= P:
        return set(range(1, t + 1))
    return set(range(1, P + 1)) | set(range(max(P + 1, t - W + 1), t + 1))


def visible(P: int, W: int, p: int, j: int) -> bool:
    """0-based form of A(t): query at position p sees key j iff j <= p and
    (j < P or j >= p - W + 1) ([PS] 03, [KV-Lean] 2.1 for the window mask)."""
    return 0 <= j <= p and (j < P or j >= p - W + 1)


def ring_to_list(buf: Sequence, head: int, count: int) -> list:
    """Read `count` entries of a ring of len(buf) slots starting at `head` ([KV-Lean] 3.4).

    The page's version reads all w slots; before the ring is full that reads
    slots that were never written ([KV-Lean] 5.1), so this reads only the
    `count` valid ones.
    """
    w = len(buf)
    return [buf[(head + i) % w] for i in range(count)]


class RingCache:
    """Physical model of the prefix-pinned cache: P prefix slots plus a W-slot ring.

    The second layer of [KV-Lean] 3.4: a fixed array with a write cursor that
    overwrites the oldest entry. `view()` reads it back as a list, and the
    tests check view() == pinned_view(P, W, history) after every push.
    """

    def __init__(self, P: int, W: int):
        if W < 1:
            raise ValueError("window must be at least 1")
        self.P, self.W = P, W
        self.prefix: list = []
        self.ring: list = [None] * W
        self.n = 0                     # tokens pushed so far

    def push(self, kv) -> None:
        if self.n < self.P:
            self.prefix.append(kv)
        else:
            self.ring[(self.n - self.P) % self.W] = kv
        self.n += 1

    def count_window(self) -> int:
        return min(self.W, max(0, self.n - self.P))

    def view(self) -> list:
        nw = self.count_window()
        head = (window_base(self.P, self.W, self.n) - self.P) % self.W
        return list(self.prefix) + ring_to_list(self.ring, head, nw)


class WindowModel:
    """List model with a per-step window length and promotion into the pinned list.

    [PS] 14 asks whether the window length could change during generation and whether
    tokens could be promoted into the pinned prefix. The reading taken here generalises
    the list model of [KV-Lean] 2.2 and 3.3 with w as a per-step parameter:

    * a token at position < P joins the pinned prefix; any other token is appended to the
      window, which then drops its oldest entries while longer than the current w;
    * set_window(w) makes w the length from now on and drops the oldest entries beyond it
      at once (dropped tokens never come back, even if w later grows);
    * promote(k) moves the k oldest window entries to the end of the pinned list, where
      they stay for good; the window keeps the rest.

    The query at the newest position attends to pinned + window.
    """

    def __init__(self, P: int, w: int):
        if w < 1:
            raise ValueError("window must be at least 1")
        self.P, self.w = P, w
        self.pinned: list = []
        self.window: list = []
        self.n = 0

    def push(self, kv) -> None:
        if self.n < self.P:
            self.pinned.append(kv)
        else:
            self.window = step(self.w, self.window, kv)
        self.n += 1

    def set_window(self, w: int) -> None:
        if w < 1:
            raise ValueError("window must be at least 1")
        self.w = w
        self.window = last_window(w, self.window)

    def promote(self, k: int) -> None:
        if k < 0 or k > len(self.window):
            raise ValueError("cannot promote more entries than the window holds")
        self.pinned = self.pinned + self.window[:k]
        self.window = self.window[k:]

    def view(self) -> list:
        return list(self.pinned) + list(self.window)
