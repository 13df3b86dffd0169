"""The float64 oracle over a pool of host processes, for whole-tensor parity at full size.

Test infrastructure (imported by GPU tests only, never by the library). Workers are
spawned, not forked: the test process has usually initialised the GPU by the time a pool is
needed, and a spawned worker starts a fresh interpreter that never touches the device (its
environment hides every GPU). Each worker runs one BLAS / torch thread. The pool holds at
most 15 workers: the GPU's share of the host is 16 cores, one of which the test process
keeps.

A job covers one sequence: the worker draws that sequence's K/V values for the union of the
visible sets of its queries once (from the seeded generator, as the oracle's history
provider would) and runs ``attn.decode_query`` on every query of the job, so a 64-step
decode or a 512-row chunk costs one draw instead of one per query. The oracle itself is
called as is.
"""
from __future__ import annotations

import hashlib
import multiprocessing as mp
import os
from typing import List, Optional, Sequence, Tuple

import numpy as np

MAX_WORKERS = 15


def n_workers() -> int:
    return max(1, min(MAX_WORKERS, len(os.sched_getaffinity(0))))


def _init_worker():
    import torch
    from threadpoolctl import threadpool_limits

    torch.set_num_threads(1)
    threadpool_limits(limits=1)


_ENV = {"OMP_NUM_THREADS": "1", "OPENBLAS_NUM_THREADS": "1", "MKL_NUM_THREADS": "1",
        "HIP_VISIBLE_DEVICES": "", "ROCR_VISIBLE_DEVICES": "", "CUDA_VISIBLE_DEVICES": ""}


class Pending:
    """Oracle jobs running in the background while the test drives the GPU."""

    def __init__(self, fn, jobs: Sequence, workers: Optional[int] = None):
        jobs = list(jobs)
        self._pool = None
        if not jobs:
            self._res = None
            return
        n = min(workers or n_workers(), len(jobs))
        saved = {k: os.environ.get(k) for k in _ENV}
        os.environ.update(_ENV)
        try:
            self._pool = mp.get_context("spawn").Pool(n, initializer=_init_worker)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v
        self._res = self._pool.map_async(fn, jobs, chunksize=1)

    def get(self) -> List:
        """The results in job order (waits for them; the pool is shut down)."""
        if self._res is None:
            return []
        try:
            return self._res.get()
        finally:
            self._pool.close()
            self._pool.join()


def run(fn, jobs: Sequence, workers: Optional[int] = None) -> List:
    """pool.map(fn, jobs) over spawned single-thread workers (results in job order)."""
    return Pending(fn, jobs, workers).get()


def _history(wl, b, positions: np.ndarray, prefix_src: Optional[int] = None):
    """Sequence b's K/V values at `positions` (sorted, unique) and a provider over them."""
    from synth import drive

    if prefix_src is None:
        base = drive.hist_provider(wl, b)
    else:
        base = drive.composite_history(wl, prefix_src, b, wl.prefix[b])
    k, v = base(positions)

    def hist(pos):
        pos = np.asarray(pos, dtype=np.int64)
        idx = np.searchsorted(positions, pos)
        assert np.array_equal(positions[idx], pos), "position outside the drawn history"
        return k[idx], v[idx]

    return hist


def decode_job(job) -> Tuple[np.ndarray, np.ndarray]:
    """job = (wl, b, positions [n], queries [n, H_q, D] float64, prefix_src or None).

    Returns (out [n, H_q, D], lse [n, H_q]) of the oracle for the queries of sequence b at
    the given absolute positions (window w_b, prefix P_b of the workload)."""
    from oracle import attn

    wl, b, positions, queries, prefix_src = job
    P, W = wl.prefix[b], wl.window_of(b)
    need = np.unique(np.concatenate([np.nonzero(attn.visible_mask(P, W, int(p)))[0]
                                     for p in positions]))
    hist = _history(wl, b, need, prefix_src)
    outs, lses = [], []
    for p, q in zip(positions, queries):
        o, s = attn.decode_query(q, int(p), hist, P, W, wl.n_kv_heads, wl.rope_base, wl.scale)
        outs.append(o)
        lses.append(s)
    return np.stack(outs), np.stack(lses)


def view_digest(pos: np.ndarray, kbits: np.ndarray, vbits: np.ndarray) -> str:
    """SHA-256 over a logical cache view: int32 positions, key bits, value bits."""
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(pos, dtype=np.int32).tobytes())
    h.update(np.ascontiguousarray(kbits).tobytes())
    h.update(np.ascontiguousarray(vbits).tobytes())
    return h.hexdigest()


def expected_view_job(job) -> Tuple[int, str]:
    """job = (wl, b, n, dtype). The list model's cache of sequence b after n tokens
    (oracle.cache.expected_view): (entry count, digest of positions, stored key bits and
    value bits). Values are stored as given, so their bits are the input's, which the
    float64 copy holds exactly (rounding it back is exact)."""
    from oracle import cache as ocache, rne
    from synth import drive

    wl, b, n, dtype = job
    pos, kbits, vref = ocache.expected_view(wl.prefix[b], wl.window_of(b), n,
                                            drive.hist_provider(wl, b), wl.rope_base, dtype)
    vbits = rne.f64_to_bf16_bits(vref) if dtype == "bf16" else rne.f64_to_f32(vref).view(np.uint32)
    return len(pos), view_digest(pos, kbits, vbits)


def whole_tensor_error(out: np.ndarray, ref: np.ndarray) -> Tuple[float, float]:
    """(max |out - ref|, ||out - ref||_2 / ||ref||_2) over the whole tensors."""
    d = out.astype(np.float64) - ref
    return float(np.abs(d).max()), float(np.linalg.norm(d) / np.linalg.norm(ref))
