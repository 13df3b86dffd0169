"""Attention forward and backward over the prefix-window mask, in row space (training).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[PS] 08: to train on long traces the trainer back-propagates either chunk by chunk,
accumulating gradients (chunked), or only through the last window with a lead context of
a few windows (truncated). Both need the gradient of attention over the same visible set
the generator used. Rows of a segment are the attended list of one sequence: rows
[0, P) are the pinned prefix, later rows are consecutive positions, so the visible set
A(t) of [PS] 03 becomes, in row indices, "key row j is visible to query row i iff
j <= i and (j < P or j >= i - W + 1)". Queries and keys arrive already rotated (the
rotation and its transpose are the trainer's), so this is plain masked attention.

Forward ([KV-Lean] 2.1 form): z_ij = scale <q_i, k_j>, -inf where masked,
p_i = softmax(z_i), o_i = sum_j p_ij v_j, lse_i = log sum_j exp(z_ij).
Backward of a loss L with dL/do_i = g_i, from the chain rule through the softmax:
  dL/dv_j = sum_i p_ij g_i
  dL/dp_ij = <g_i, v_j>
  dL/dz_ij = p_ij (dL/dp_ij - sum_l p_il dL/dp_il) = p_ij (<g_i, v_j> - <g_i, o_i>)
  dL/dq_i = scale sum_j dL/dz_ij k_j,   dL/dk_j = scale sum_i dL/dz_ij q_i
With grouped-query heads, a key/value head's gradient sums over the query heads that
read it (query head hq reads KV head hq // (H_q / H_kv)).
All arithmetic in float64.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np


def row_mask(T: int, P: int, W: int) -> np.ndarray:
    """[T, T] boolean: query row i sees key row j."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    return (j <= i) & ((j < P) | (j >= i - W + 1))


def forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, P: int, W: int, scale: float
            ) -> Tuple[np.ndarray, np.ndarray]:
    """q [T, H_q, D], k, v [T, H_kv, D] -> (out [T, H_q, D], lse [T, H_q])."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    mask = row_mask(T, P, W)
    out = np.empty((T, Hq, D))
    lse = np.empty((T, Hq))
    for hq in range(Hq):
        hk = hq // G
        z = np.where(mask, scale * (q[:, hq, :] @ k[:, hk, :].T), -np.inf)
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)                  # exactly 0 where masked
        s = e.sum(axis=1, keepdims=True)
        out[:, hq, :] = (e / s) @ v[:, hk, :]
        lse[:, hq] = (m + np.log(s))[:, 0]
    return out, lse


def backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, dout: np.ndarray, P: int, W: int,
             scale: float) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients (dq [T, H_q, D], dk, dv [T, H_kv, D]) of a loss with dL/dout = dout."""
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    mask = row_mask(T, P, W)
    dq = np.zeros_like(q)
    dk = np.zeros((T, Hkv, D))
    dv = np.zeros((T, Hkv, D))
    for hq in range(Hq):
        hk = hq // G
        z = np.where(mask, scale * (q[:, hq, :] @ k[:, hk, :].T), -np.inf)
        e = np.exp(z - z.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ v[:, hk, :]
        dp = g[:, hq, :] @ v[:, hk, :].T
        dz = p * (dp - np.sum(g[:, hq, :] * o, axis=1, keepdims=True))
        dv[:, hk, :] += p.T @ g[:, hq, :]
        dq[:, hq, :] = scale * (dz @ k[:, hk, :])
        dk[:, hk, :] += scale * (dz.T @ q[:, hq, :])
    return dq, dk, dv


def visible_keys(i: int, P: int, W: int) -> np.ndarray:
    """Key rows visible to query row i: [0, min(P, i + 1)) and [max(P, i - W + 1), i]."""
    return np.concatenate([np.arange(min(P, i + 1)), np.arange(max(P, i - W + 1), i + 1)])


def seeing_rows(j: int, T: int, P: int, W: int) -> np.ndarray:
    """Query rows that see key row j: every later row for a prefix key, else [j, j + W)."""
    return np.arange(j, T) if j < P else np.arange(j, min(T, j + W))


def _row(q, k, v, g, i, hq, G, P, W, scale):
    """Row i, query head hq over its visible keys (two contiguous row ranges, read as
    slices): (ranges, p, o, lse, dz) with dz = p (dp - <g_i, o_i>) when g is given."""
    hk = hq // G
    ranges = [(0, min(P, i + 1)), (max(P, i - W + 1), i + 1)]
    z = np.concatenate([scale * (k[a:b, hk, :] @ q[i, hq, :]) for a, b in ranges])
    m = z.max()
    e = np.exp(z - m)
    p = e / e.sum()
    n0 = ranges[0][1]
    o = p[:n0] @ v[0:n0, hk, :] + p[n0:] @ v[ranges[1][0]:ranges[1][1], hk, :]
    dz = None
    if g is not None:
        dp = np.concatenate([v[a:b, hk, :] @ g[i, hq, :] for a, b in ranges])
        dz = p * (dp - g[i, hq, :] @ o)
    return ranges, p, o, m + np.log(e.sum()), dz


def _index(ranges, j):
    """Where key row j sits in the concatenation of the two ranges."""
    (a0, b0), (a1, _) = ranges
    return j - a0 if j < b0 else (b0 - a0) + (j - a1)


def forward_rows(q, k, v, P: int, W: int, scale: float, rows) -> Tuple[np.ndarray, np.ndarray]:
    """`forward` at the listed query rows only, each from its own visible keys (large T)."""
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    Hq, G = q.shape[1], q.shape[1] // k.shape[1]
    out = np.empty((len(rows), Hq, q.shape[2]))
    lse = np.empty((len(rows), Hq))
    for r, i in enumerate(rows):
        for hq in range(Hq):
            _, _, out[r, hq], lse[r, hq], _ = _row(q, k, v, None, i, hq, G, P, W, scale)
    return out, lse


def backward_rows(q, k, v, dout, P: int, W: int, scale: float, q_rows, k_rows
                  ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """`backward` at the listed rows only: dq at q_rows, dk and dv at k_rows.

    dq_i needs row i's probabilities; dk_j and dv_j sum over the rows that see j, each
    with its full row softmax and sum_l p_il dL/dp_il. Same formulas as `backward`,
    evaluated row by row so that only the rows involved are touched.
    """
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros((len(q_rows), Hq, D))
    for r, i in enumerate(q_rows):
        for hq in range(Hq):
            ranges, _, _, _, dz = _row(q, k, v, g, i, hq, G, P, W, scale)
            n0 = ranges[0][1]
            dq[r, hq] = scale * (dz[:n0] @ k[0:n0, hq // G, :] +
                                 dz[n0:] @ k[ranges[1][0]:ranges[1][1], hq // G, :])
    dk = np.zeros((len(k_rows), Hkv, D))
    dv = np.zeros((len(k_rows), Hkv, D))
    for r, j in enumerate(k_rows):
        for hq in range(Hq):
            hk = hq // G
            for i in seeing_rows(j, T, P, W):
                ranges, p, _, _, dz = _row(q, k, v, g, i, hq, G, P, W, scale)
                at = _index(ranges, j)
                dv[r, hk] += p[at] * g[i, hq]
                dk[r, hk] += scale * dz[at] * q[i, hq]
    return dq, dk, dv
