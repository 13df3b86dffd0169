"""Feed synthetic workloads through the library (tests and benchmark).

Inputs only: this module generates the seeded K/V/Q values with `synth.gen` and
hands them to the library's calls; it computes nothing of the method itself.
"""
from __future__ import annotations

from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import gen
from .configs import Workload


def hist_provider(wl: Workload, b: int) -> Callable[[np.ndarray], Tuple[np.ndarray, np.ndarray]]:
    """History of sequence b as the oracle wants it: pos -> (k, v) float64 [n, H_kv, D]."""
    def hist(pos):
        pos = torch.as_tensor(np.asarray(pos, dtype=np.int64))
        width = wl.n_kv_heads * wl.head_dim
        k = gen.normal_at(wl.seed, gen.STREAM_K, b, pos, width, wl.dtype)
        v = gen.normal_at(wl.seed, gen.STREAM_V, b, pos, width, wl.dtype)
        shape = (-1, wl.n_kv_heads, wl.head_dim)
        return k.double().numpy().reshape(shape), v.double().numpy().reshape(shape)
    return hist


def composite_history(wl: Workload, prefix_src: int, window_src: int, P: int):
    """History whose positions < P come from sequence prefix_src's values and the rest from
    window_src's (a sequence reading a prefix written from another sequence's values)."""
    pre = hist_provider(wl, prefix_src)
    own = hist_provider(wl, window_src)

    def hist(pos):
        pos = np.asarray(pos, dtype=np.int64)
        k1, v1 = pre(pos)
        k2, v2 = own(pos)
        sel = (pos < P)[:, None, None]
        return np.where(sel, k1, k2), np.where(sel, v1, v2)
    return hist


def kv_rows_from(wl: Workload, src_seqs: Sequence[int], starts: Sequence[int], n: int, device="cpu"
                 ) -> Tuple[torch.Tensor, torch.Tensor]:
    """k, v [len(src_seqs), n, H_kv, D]: row r holds sequence src_seqs[r]'s values at
    positions starts[r] .. starts[r] + n - 1."""
    k = gen.normal_block(wl.seed, gen.STREAM_K, list(src_seqs), list(starts), n, wl.n_kv_heads,
                         wl.head_dim, wl.dtype, device)
    v = gen.normal_block(wl.seed, gen.STREAM_V, list(src_seqs), list(starts), n, wl.n_kv_heads,
                         wl.head_dim, wl.dtype, device)
    return k, v


def queries(wl: Workload, positions: Sequence[int], device="cpu", seqs=None) -> torch.Tensor:
    """q of the token at positions[b] for each sequence: [len(seqs), H_q, D]."""
    seqs = list(range(wl.batch)) if seqs is None else list(seqs)
    pos = torch.as_tensor([int(p) for p in positions], dtype=torch.int64)
    q = gen.normal_at(wl.seed, gen.STREAM_Q, torch.as_tensor(seqs), pos,
                      wl.n_q_heads * wl.head_dim, wl.dtype, device)
    return q.view(len(seqs), wl.n_q_heads, wl.head_dim)


def query_block(wl: Workload, starts: Sequence[int], n: int, device="cpu") -> torch.Tensor:
    """q rows for positions starts[b] .. starts[b] + n - 1: [B, n, H_q, D]."""
    return gen.normal_block(wl.seed, gen.STREAM_Q, list(range(wl.batch)), list(starts), n,
                            wl.n_q_heads, wl.head_dim, wl.dtype, device)


def kv_block(wl: Workload, starts: Sequence[int], n: int, device="cpu"
             ) -> Tuple[torch.Tensor, torch.Tensor]:
    """k, v rows for positions starts[b] .. starts[b] + n - 1: [B, n, H_kv, D] each."""
    bs = list(range(wl.batch))
    k = gen.normal_block(wl.seed, gen.STREAM_K, bs, list(starts), n, wl.n_kv_heads, wl.head_dim,
                         wl.dtype, device)
    v = gen.normal_block(wl.seed, gen.STREAM_V, bs, list(starts), n, wl.n_kv_heads, wl.head_dim,
                         wl.dtype, device)
    return k, v


def make_cache(wl: Workload, max_chunk: int = 0, device="cuda", n_shared: int = 0,
               shared_max: int = 0, prefix_max: Optional[int] = None, pe: str = "continue",
               block_size: int = 0, n_blocks: int = 0):
    import prefix_pinned_sliding_amd as psa
    pmax = wl.prefix_max if prefix_max is None else prefix_max
    return psa.Cache(wl.batch, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, pmax,
                     wl.window, wl.dtype, wl.rope_base, 0.0, max_chunk, device=device,
                     n_shared_prefixes=n_shared, shared_prefix_max=shared_max, pe=pe,
                     block_size=block_size, n_blocks=n_blocks)


def fill(cache, wl: Workload, n_hist: List[int], device="cuda", chunk: Optional[int] = None,
         reset: bool = True) -> None:
    """Reset every sequence with its prefix length and append positions [0, n_hist[b]).

    Values are generated only for sequences that still take tokens in a chunk; the rows
    of the others are left unset and passed with a count of 0.
    """
    B = wl.batch
    if reset:
        for b in range(B):
            cache.reset(b, wl.prefix[b])
            if wl.windows is not None:
                cache.set_window(b, wl.windows[b])
    maxn = max(n_hist) if n_hist else 0
    if chunk is None:
        per_pos = B * wl.n_kv_heads * wl.head_dim
        chunk = max(256, min(8192, (1 << 27) // per_pos))
    ragged = len(set(n_hist)) > 1
    for p0 in range(0, maxn, chunk):
        n = min(chunk, maxn - p0)
        counts = [min(max(nb - p0, 0), n) for nb in n_hist]
        active = [b for b in range(B) if counts[b] > 0]
        if len(active) == B:
            k, v = kv_block(wl, [p0] * B, n, device)
        else:
            shape = (B, n, wl.n_kv_heads, wl.head_dim)
            k = torch.empty(shape, dtype=wl.dtype, device=device)
            v = torch.empty_like(k)
            k[active] = gen.normal_block(wl.seed, gen.STREAM_K, active, [p0] * len(active), n,
                                         wl.n_kv_heads, wl.head_dim, wl.dtype, device)
            v[active] = gen.normal_block(wl.seed, gen.STREAM_V, active, [p0] * len(active), n,
                                         wl.n_kv_heads, wl.head_dim, wl.dtype, device)
        cache.append(k, v, n_new=counts if ragged else None)
    torch.cuda.synchronize()


def fill_one_prompt(cache, wl: Workload, n_hist: List[int], shared: bool, device="cuda",
                    chunk: Optional[int] = None) -> None:
    """Every sequence runs the same prompt: positions < P hold sequence 0's values, later
    positions the sequence's own. With `shared` the prompt is written once into pool entry
    0 and every sequence attaches to it; otherwise each sequence appends its own copy."""
    B, P = wl.batch, wl.prefix[0]
    kp, vp = kv_rows_from(wl, [0], [0], P, device)
    if shared:
        cache.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())
        for b in range(B):
            cache.attach(b, 0)
    else:
        for b in range(B):
            cache.reset(b, P)
        cache.append(kp.expand(B, -1, -1, -1).contiguous(), vp.expand(B, -1, -1, -1).contiguous())
    maxn = max(n_hist)
    if chunk is None:
        chunk = max(256, min(8192, (1 << 27) // (B * wl.n_kv_heads * wl.head_dim)))
    for p0 in range(P, maxn, chunk):
        n = min(chunk, maxn - p0)
        k, v = kv_block(wl, [p0] * B, n, device)
        cache.append(k, v)
    torch.cuda.synchronize()
