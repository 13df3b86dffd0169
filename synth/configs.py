"""The synthetic workloads the path is tested and measured on.

Shapes only, plus the seeded per-sequence draws of prefix lengths and start
positions. "At t" is the 1-based position of the first new token, so the
cache holds positions [0, t - 1) before it is appended (0-based p = t - 1).

The pages' own workloads (reasoning traces of a 1.7B model with W = 4096 and
a prompt as the pinned prefix, up to 262,144 generated tokens) are not
available; these shapes stand in for them, with N(0,1) values from `synth.gen`.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch


@dataclasses.dataclass
class Workload:
    name: str
    dtype: torch.dtype
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    window: int
    prefix: List[int]          # P_b per sequence
    start: List[int]           # 1-based t_b of the first new token per sequence
    kind: str                  # "decode" or "prefill"
    steps: int = 1             # decode steps (append + decode) per run
    chunk: int = 0             # prefill chunk length
    rope_base: float = 10000.0
    seed: int = 0
    windows: Optional[List[int]] = None   # per-sequence window lengths (None: all `window`)

    @property
    def prefix_max(self) -> int:
        return max(self.prefix)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def window_of(self, b: int) -> int:
        return self.window if self.windows is None else self.windows[b]



def tiny_fp32(seed: int = 0) -> Workload:
    """fp32, batch 1, 4/4 heads, D=64, P=16, W=32, 200 decode steps from an empty cache."""
    return Workload("tiny-fp32-P16-W32", torch.float32, 1, 4, 4, 64, 32, [16], [1],
                    "decode", steps=200, seed=seed)


def decode_p100_w4096(seed: int = 0, batch: int = 64, t: int = 32768) -> Workload:
    """bf16, 64 sequences at t=32768, 16/8 heads, D=128, P=100, W=4096, one decode step."""
    return Workload(f"decode-bf16-B{batch}-P100-W4096-t{t}", torch.bfloat16, batch, 16, 8, 128,
                    4096, [100] * batch, [t] * batch, "decode", steps=1, seed=seed)


def prefill_chunk512(seed: int = 0, batch: int = 8) -> Workload:
    """bf16, 8 sequences each appending a 512-token chunk at t ~ U{8192..65536}."""
    rng = np.random.Generator(np.random.PCG64(seed))
    starts = [int(x) for x in rng.integers(8192, 65536, size=batch, endpoint=True)]
    return Workload(f"prefill-bf16-B{batch}-P100-W4096-C512", torch.bfloat16, batch, 16, 8, 128,
                    4096, [100] * batch, starts, "prefill", chunk=512, seed=seed)


def decode_p512_w16384(seed: int = 0, batch: int = 32, t: int = 100000) -> Workload:
    """bf16, 32 sequences at t=100000, 32/8 heads, D=128, P=512, W=16384."""
    return Workload(f"decode-bf16-B{batch}-P512-W16384-t{t}", torch.bfloat16, batch, 32, 8, 128,
                    16384, [512] * batch, [t] * batch, "decode", steps=1, seed=seed)


def ragged_decode(seed: int = 0, batch: int = 256, steps: int = 64) -> Workload:
    """bf16, 256 sequences, P_b ~ U{50..2000}, t_b ~ floor(exp(U(ln 1000, ln 131072))), 64 steps."""
    rng = np.random.Generator(np.random.PCG64(seed + 5))
    prefix = [int(x) for x in rng.integers(50, 2000, size=batch, endpoint=True)]
    u = rng.uniform(math.log(1000.0), math.log(131072.0), size=batch)
    starts = [int(math.floor(math.exp(x))) for x in u]
    return Workload(f"ragged-decode-bf16-B{batch}-W4096", torch.bfloat16, batch, 16, 8, 128,
                    4096, prefix, starts, "decode", steps=steps, seed=seed)


def decode_shared_p2000(seed: int = 0, batch: int = 64, t: int = 32768) -> Workload:
    """bf16, 64 runs of one prompt: a 2000-token prefix (sequence 0's values for every run),
    W=4096, t=32768, 16/8 heads, D=128. Used with the prefix shared or copied per run."""
    return Workload(f"decode-bf16-B{batch}-P2000shared-W4096-t{t}", torch.bfloat16, batch, 16, 8,
                    128, 4096, [2000] * batch, [t] * batch, "decode", steps=1, seed=seed)


def decode_ragged_window(seed: int = 0, batch: int = 64, t: int = 32768) -> Workload:
    """bf16, 64 sequences at t=32768, 16/8 heads, D=128, P=100, ring of 4096 slots and a
    window length per sequence w_b ~ U{256..4096}."""
    rng = np.random.Generator(np.random.PCG64(seed + 11))
    wins = [int(x) for x in rng.integers(256, 4096, size=batch, endpoint=True)]
    return Workload(f"decode-bf16-B{batch}-P100-Wragged256to4096-t{t}", torch.bfloat16, batch, 16,
                    8, 128, 4096, [100] * batch, [t] * batch, "decode", steps=1, seed=seed,
                    windows=wins)


ALL = {
    "tiny_fp32": tiny_fp32,
    "decode_p100_w4096": decode_p100_w4096,
    "prefill_chunk512": prefill_chunk512,
    "decode_p512_w16384": decode_p512_w16384,
    "ragged_decode": ragged_decode,
    "decode_shared_p2000": decode_shared_p2000,
    "decode_ragged_window": decode_ragged_window,
}


def by_name(name: str, **kw) -> Workload:
    return ALL[name](**kw)
