"""Attention reference: full history, -inf outside the visible set, float64 softmax.

TEST INFRASTRUCTURE ONLY (see the package docstring).

[KV-Lean] 2.1 defines the reference model: the query attends over the whole
history with logits q K^T / sqrt(d) plus a window mask (-inf for positions
older than the window) and a causal mask. [PS] 03 widens the window mask to
keep the pinned prefix: the query at 1-based t sees [1, P] and
[max(P + 1, t - W + 1), t]. [KV-Lean] 1.1 and 4.2 note that a masked
position has softmax weight exactly 0, which is why a bounded cache can be
exact.

Inputs are the values as stored in the input tensors (queries, keys and
values in the input dtype, converted exactly to float64). Queries and keys
are rotated here in float64 at their absolute positions (unrounded), so the
only roundings are float64 ones.

History providers: ``hist(positions) -> (k, v)`` returns float64 arrays
[len(positions), H_kv, D] for any set of absolute positions of one sequence.
That lets the reference "keep the whole unbounded history" without ever
materialising positions whose logit is -inf.
"""
from __future__ import annotations

from typing import Callable, Tuple

import numpy as np

from . import rope, spec

History = Callable[[np.ndarray], Tuple[np.ndarray, np.ndarray]]


def visible_mask(P: int, W: int, p: int) -> np.ndarray:
    """Boolean mask over keys j = 0..p of the query at 0-based position p.

    Visible iff j < P (pinned prefix) or j >= p - W + 1 (window); every j
    here is <= p (causal). This is A(t) of [PS] 03 with t = p + 1.
    """
    j = np.arange(p + 1)
    return (j < P) | (j >= p - W + 1)


def _softmax_attend(logits: np.ndarray, vals: np.ndarray, rows=None) -> Tuple[np.ndarray, float]:
    """softmax(logits) @ vals plus the log-sum-exp, for logits that may hold -inf.

    exp(-inf - m) is exactly 0, so the weighted sum may skip those rows:
    `rows` (optional) selects the logit entries that `vals` holds, in order.
    """
    m = np.max(logits)
    w = np.exp(logits - m)            # exactly 0 where the logit is -inf
    l = np.sum(w)
    wv = w if rows is None else w[rows]
    return (wv @ vals) / l, float(m + np.log(l))


def reset_positions(P: int, W: int, p: int, keys: np.ndarray) -> Tuple[int, np.ndarray]:
    """Positions under Reset PE ([PS] 05): the attended tokens are renumbered as one
    contiguous sequence, prefix first, window after it.

    The reading taken here: the model sees the cache list [prefix, window] as positions
    0 .. len - 1, so prefix token j keeps position j and window token j (absolute) gets
    P + (j - base) with base = max(P, p - W + 1) the oldest window position; the query
    (the newest window token) gets P + (p - base). Inside the prefix (p < P) nothing
    moves. Returns (query position, key positions).
    """
    keys = np.asarray(keys, dtype=np.int64)
    if p < P:
        return p, keys
    base = max(P, p - W + 1)
    return P + (p - base), np.where(keys < P, keys, P + (keys - base))


def decode_query(q: np.ndarray, p: int, hist: History, P: int, W: int, n_kv_heads: int,
                 base: float, scale: float, pe: str = "continue") -> Tuple[np.ndarray, np.ndarray]:
    """Attention of one token's queries q[H_q, D] at absolute position p.

    Builds the length-(p+1) logit vector of every query head, -inf where the
    mask says the key is not visible, and runs the softmax over it. Only the
    visible keys and values are fetched from `hist`: a masked logit is -inf
    whatever its key holds. Query head hq reads KV head hq // (H_q / H_kv)
    (contiguous groups; the pages do not discuss grouped-query heads).

    `pe` = "continue" rotates every token at its absolute position ([PS] 05, the method's
    choice); "reset" rotates at the positions of `reset_positions`.

    Returns (out[H_q, D], lse[H_q]) in float64; lse is the natural-log
    log-sum-exp of the scaled logits.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    G = Hq // n_kv_heads
    mask = visible_mask(P, W, p)
    pos = np.nonzero(mask)[0]
    k, v = hist(pos)
    qpos, kpos = (p, pos) if pe == "continue" else reset_positions(P, W, p, pos)
    qr = rope.rotate(q, np.full(Hq, qpos), base)
    kr = rope.rotate(k, np.broadcast_to(kpos[:, None], k.shape[:2]), base)
    out = np.empty((Hq, D))
    lse = np.empty(Hq)
    for hq in range(Hq):
        hk = hq // G
        logits = np.full(p + 1, -np.inf)
        logits[mask] = (kr[:, hk, :] @ qr[hq]) * scale
        out[hq], lse[hq] = _softmax_attend(logits, v[:, hk, :], rows=mask)
    return out, lse


def decode_query_from_cache(q: np.ndarray, p: int, hist: History, P: int, W: int,
                            n_kv_heads: int, base: float, scale: float
                            ) -> Tuple[np.ndarray, np.ndarray]:
    """The same attention computed over the list-model cache instead of a mask.

    The cache after tokens 0..p is pinned_view(P, W, [0..p]) (the prefix plus
    the last window); attention over exactly its entries equals attention over
    the full history with the mask ([KV-Lean] 4.2: out-of-window weights are
    zero). Agreement of the two functions ties the mask to the cache model.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    G = Hq // n_kv_heads
    pos = np.asarray(spec.pinned_view(P, W, range(p + 1)), dtype=np.int64)
    k, v = hist(pos)
    qr = rope.rotate(q, np.full(Hq, p), base)
    kr = rope.rotate(k, np.broadcast_to(pos[:, None], k.shape[:2]), base)
    out = np.empty((Hq, D))
    lse = np.empty(Hq)
    for hq in range(Hq):
        hk = hq // G
        logits = (kr[:, hk, :] @ qr[hq]) * scale
        out[hq], lse[hq] = _softmax_attend(logits, v[:, hk, :])
    return out, lse


def attend_view(q: np.ndarray, p: int, hist: History, view, n_kv_heads: int, base: float,
                scale: float, pe: str = "continue") -> Tuple[np.ndarray, np.ndarray]:
    """Attention of the query at position p over an explicit cache list.

    `view` is the list model's cache after token p, in list order (pinned entries, then
    the window, oldest first), as absolute positions; spec.WindowModel gives it for
    caches that are not a closed-form set (a window whose length changed, promoted
    tokens). Every position not in the list has logit -inf ([KV-Lean] 2.1: masked
    positions get zero weight), so only the listed ones are fetched.

    "continue" rotates at absolute positions. "reset" ([PS] 05) renumbers the attended
    list as one sequence: entry i of `view` gets position i and the query, the newest
    entry, len(view) - 1; on the closed-form set this is `reset_positions`.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, D = q.shape
    G = Hq // n_kv_heads
    pos = np.asarray(list(view), dtype=np.int64)
    k, v = hist(pos)
    if pe == "continue":
        qpos, kpos = p, pos
    else:
        qpos, kpos = len(pos) - 1, np.arange(len(pos))
    qr = rope.rotate(q, np.full(Hq, qpos), base)
    kr = rope.rotate(k, np.broadcast_to(kpos[:, None], k.shape[:2]), base)
    out = np.empty((Hq, D))
    lse = np.empty(Hq)
    for hq in range(Hq):
        hk = hq // G
        logits = np.full(p + 1, -np.inf)
        logits[pos] = (kr[:, hk, :] @ qr[hq]) * scale
        out[hq], lse[hq] = _softmax_attend(logits, v[:, hk, :], rows=pos)
    return out, lse


def prefill_chunk(q: np.ndarray, n: int, hist: History, P: int, W: int, n_kv_heads: int,
                  base: float, scale: float, rows=None, pe: str = "continue"
                  ) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of a chunk of queries q[C, H_q, D] at positions n .. n + C - 1.

    Each query at p sees A(p + 1) over the history including the chunk's own
    tokens up to p. The pages never discuss chunks; the reading is that a
    chunk is the same as C consecutive single-token steps, so `hist` must
    cover positions up to n + C - 1. `rows` picks a subset of chunk rows
    (default all). Returns (out[len(rows), H_q, D], lse[len(rows), H_q]).
    """
    C = q.shape[0]
    rows = range(C) if rows is None else rows
    outs, lses = [], []
    for c in rows:
        o, s = decode_query(q[c], n + c, hist, P, W, n_kv_heads, base, scale, pe)
        outs.append(o)
        lses.append(s)
    return np.stack(outs), np.stack(lses)


def array_history(k: np.ndarray, v: np.ndarray) -> History:
    """A history provider over explicit arrays k, v [n, H_kv, D] (position = row)."""
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)

    def hist(pos):
        pos = np.asarray(pos, dtype=np.int64)
        return k[pos], v[pos]

    return hist
