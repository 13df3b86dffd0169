"""Seeded, counter-based synthetic inputs.

This module is shared by the tests, the oracle checks and the benchmark, and
by nothing else. It holds none of the attention method's arithmetic: it only
maps (seed, stream, sequence, position, element) to a number.

Generator. Every value is one output of SplitMix64 (G. Steele, D. Lea,
C. Flood, "Fast splittable pseudorandom number generators", OOPSLA 2014):
the output with counter c of a stream keyed by k is ``mix(k + c * GAMMA)``
modulo 2**64, with the published GAMMA and the published 64-bit finaliser
``mix``. Because the value of element i of position p depends only on
(seed, stream, b, p, i), any position of any sequence can be regenerated on
its own, which is what lets the oracle look at the visible positions of a
100k-token history without generating the rest.

Distribution. The top 16 bits of the output index a table of the 65536
N(0,1) quantiles Phi^-1((j + 1/2) / 65536), so values follow N(0,1) up to
that quantisation (tails cut at about 4.33). The table is built once on the
CPU in float64 and rounded to the requested dtype there, so every device
produces bit-identical tensors: the generator uses only integer arithmetic
and a table gather.

All arithmetic is on torch int64 (wrapping two's-complement products give the
same low 64 bits as unsigned ones; right shifts are made logical by masking).
"""
from __future__ import annotations

import functools

import numpy as np
import torch

STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3
STREAM_DO = 4   # output gradients of the training workloads

_M64 = 1 << 64


def _i64(c: int) -> int:
    """Reinterpret an unsigned 64-bit constant as a signed int64."""
    return c - _M64 if c >= (1 << 63) else c


GAMMA = _i64(0x9E3779B97F4A7C15)
_C1 = _i64(0xBF58476D1CE4E5B9)
_C2 = _i64(0x94D049BB133111EB)


def _srl(x: torch.Tensor, s: int) -> torch.Tensor:
    """Logical right shift of an int64 tensor."""
    return (x >> s) & ((1 << (64 - s)) - 1)


def mix(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 finaliser on int64 tensors (bitwise equal to the uint64 one)."""
    z = (z ^ _srl(z, 30)) * _C1
    z = (z ^ _srl(z, 27)) * _C2
    return z ^ _srl(z, 31)


def mix_int(z: int) -> int:
    """The same finaliser on Python ints modulo 2**64 (used to pin `mix`)."""
    z %= _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) % _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) % _M64
    return z ^ (z >> 31)


def stream_key(seed: int, stream: int, b: torch.Tensor) -> torch.Tensor:
    """Key of the (seed, stream, sequence b) stream, as int64."""
    k0 = mix(torch.tensor(_i64((seed * 0x9E3779B97F4A7C15 + 0x632BE59BD9B4E019) % _M64),
                          dtype=torch.int64))
    k1 = mix(k0 + torch.tensor(stream, dtype=torch.int64) * GAMMA)
    return mix(k1.to(b.device) + b.to(torch.int64) * GAMMA)


@functools.lru_cache(maxsize=None)
def _table_cpu(dtype: torch.dtype) -> torch.Tensor:
    from scipy.special import ndtri

    j = np.arange(65536, dtype=np.float64)
    q = ndtri((j + 0.5) / 65536.0)
    return torch.from_numpy(q).to(dtype)


_table_dev: dict = {}


def quantile_table(dtype: torch.dtype, device) -> torch.Tensor:
    """The 65536-entry N(0,1) quantile table in `dtype` on `device`."""
    device = torch.device(device)
    key = (dtype, str(device))
    if key not in _table_dev:
        _table_dev[key] = _table_cpu(dtype).to(device)
    return _table_dev[key]


def normal_at(seed: int, stream: int, b, p, width: int,
              dtype: torch.dtype = torch.float32, device="cpu") -> torch.Tensor:
    """N(0,1) values for sequences `b` and positions `p` (broadcast together).

    Returns a tensor of shape broadcast(b, p).shape + (width,). Element i of
    position p of sequence b is the SplitMix64 output with counter
    p * width + i + 1 of the (seed, stream, b) stream, mapped through the
    quantile table.
    """
    device = torch.device(device)
    b = torch.as_tensor(b, dtype=torch.int64, device=device)
    p = torch.as_tensor(p, dtype=torch.int64, device=device)
    b, p = torch.broadcast_tensors(b, p)
    key = stream_key(seed, stream, b)                          # [...]
    i = torch.arange(width, dtype=torch.int64, device=device)
    ctr = p.unsqueeze(-1) * width + i + 1                      # [..., width]
    z = mix(key.unsqueeze(-1) + ctr * GAMMA)
    idx = _srl(z, 48)
    return quantile_table(dtype, device)[idx]


def normal_rows(seed: int, stream: int, b: int, p0: int, p1: int, heads: int, head_dim: int,
                dtype: torch.dtype = torch.float32, device="cpu") -> torch.Tensor:
    """Rows for positions [p0, p1) of sequence b, shaped [p1 - p0, heads, head_dim]."""
    p = torch.arange(p0, p1, dtype=torch.int64)
    out = normal_at(seed, stream, b, p, heads * head_dim, dtype, device)
    return out.view(p1 - p0, heads, head_dim)


def normal_block(seed: int, stream: int, bs, p_start, n: int, heads: int, head_dim: int,
                 dtype: torch.dtype = torch.float32, device="cpu") -> torch.Tensor:
    """A [len(bs), n, heads, head_dim] block: row j of sequence bs[r] is position p_start[r] + j."""
    device = torch.device(device)
    bs = torch.as_tensor(bs, dtype=torch.int64, device=device)
    p_start = torch.as_tensor(p_start, dtype=torch.int64, device=device)
    p = p_start.view(-1, 1) + torch.arange(n, dtype=torch.int64, device=device).view(1, -1)
    out = normal_at(seed, stream, bs.view(-1, 1), p, heads * head_dim, dtype, device)
    return out.view(bs.numel(), n, heads, head_dim)
