"""Python binding of libpsa (prefix-pinned sliding-window attention for MI355X).

Argument marshalling only: torch tensors supply device memory and the HIP stream,
and every call goes straight to the C-ABI in ``libpsa.so`` (declared in
``include/psa.h``). There is no fallback: importing this package raises if the
library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpsa.so")

PSA_OK, PSA_ERR_ARG, PSA_ERR_STATE, PSA_ERR_OVERFLOW, PSA_ERR_HIP = 0, 1, 2, 3, 4
PSA_BF16, PSA_F32 = 0, 1
PSA_PE_CONTINUE, PSA_PE_RESET = 0, 1
_PE = {"continue": PSA_PE_CONTINUE, "reset": PSA_PE_RESET}
K_APPEND, K_DECODE, K_MERGE, K_PREFILL_STAGE, K_PREFILL = 0, 1, 2, 3, 4
KERNEL_NAMES = {K_APPEND: "append", K_DECODE: "decode_partial", K_MERGE: "merge",
                K_PREFILL_STAGE: "prefill_stage", K_PREFILL: "prefill"}

_DTYPES = {torch.bfloat16: PSA_BF16, torch.float32: PSA_F32}


class Desc(ctypes.Structure):
    """psa_cache_desc."""
    _fields_ = [
        ("max_batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("prefix_max", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("max_chunk", ctypes.c_int32),
        ("rope_base", ctypes.c_double),
        ("scale", ctypes.c_float),
        ("n_shared_prefixes", ctypes.c_int32),
        ("shared_prefix_max", ctypes.c_int32),
        ("pe_mode", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
    ]


class Layout(ctypes.Structure):
    """psa_layout."""
    _fields_ = [
        ("k_offset", ctypes.c_size_t),
        ("v_offset", ctypes.c_size_t),
        ("pool_k_offset", ctypes.c_size_t),
        ("pool_v_offset", ctypes.c_size_t),
        ("tags_offset", ctypes.c_size_t),
        ("btab_offset", ctypes.c_size_t),
        ("state_offset", ctypes.c_size_t),
        ("work_offset", ctypes.c_size_t),
        ("total_bytes", ctypes.c_size_t),
        ("slots", ctypes.c_int32),
        ("elem_bytes", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("n_blocks", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
    ]


class TrainDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("seq_len", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("reserved", ctypes.c_int32),
    ]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m prefix_pinned_sliding_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sigs = {
        "psa_cache_bytes": (SZ, [ctypes.POINTER(Desc)]),
        "psa_cache_layout": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Layout)]),
        "psa_cache_create": (ctypes.c_int, [ctypes.POINTER(Desc), P, SZ, P, ctypes.POINTER(P)]),
        "psa_cache_destroy": (ctypes.c_int, [P]),
        "psa_seq_reset": (ctypes.c_int, [P, I32, I32, P]),
        "psa_prefix_load": (ctypes.c_int, [P, I32, I32, P, P, P]),
        "psa_seq_attach": (ctypes.c_int, [P, I32, I32, P]),
        "psa_seq_set_window": (ctypes.c_int, [P, I32, I32, P]),
        "psa_seq_promote": (ctypes.c_int, [P, I32, I32, P]),
        "psa_seq_window": (ctypes.c_int, [P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32),
                                          ctypes.POINTER(I32)]),
        "psa_seq_blocks": (ctypes.c_int, [P, I32, P, ctypes.POINTER(I32), ctypes.POINTER(I32)]),
        "psa_append": (ctypes.c_int, [P, P, I32, P, P, I32, P]),
        "psa_decode_attn": (ctypes.c_int, [P, P, P, P, P]),
        "psa_decode_step": (ctypes.c_int, [P, P, P, P, P, P, P]),
        "psa_prefill_attn": (ctypes.c_int, [P, I32, P, P, P, P, P, P]),
        "psa_export": (ctypes.c_int, [P, I32, P, P, P, ctypes.POINTER(I32), P]),
        "psa_seq_length": (I64, [P, I32]),
        "psa_set_split_tokens": (ctypes.c_int, [P, I32]),
        "psa_profile": (ctypes.c_int, [P, I32]),
        "psa_profile_read": (ctypes.c_int, [P, I32, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(I64)]),
        "psa_train_workspace_bytes": (SZ, [ctypes.POINTER(TrainDesc)]),
        "psa_train_fwd": (ctypes.c_int, [ctypes.POINTER(TrainDesc), P, P, P, P, P, P, P, P, SZ, P]),
        "psa_train_bwd": (ctypes.c_int, [ctypes.POINTER(TrainDesc), P, P, P, P, P, P, P, P, P, P,
                                         P, P, SZ, P]),
        "psa_train_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(TrainDesc), P, P, P, P, P, P, P,
                                                 P, P, P, P, P]),
        "psa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "psa_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class PsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.psa_last_error().decode()
        super().__init__(f"{where}: {lib.psa_status_string(status).decode()} ({msg})")


def _check(status: int, where: str) -> None:
    if status != PSA_OK:
        raise PsaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def make_desc(max_batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int, prefix_max: int,
              window: int, dtype: torch.dtype = torch.bfloat16, rope_base: float = 10000.0,
              scale: float = 0.0, max_chunk: int = 0, n_shared_prefixes: int = 0,
              shared_prefix_max: int = 0, pe: str = "continue", block_size: int = 0,
              n_blocks: int = 0) -> Desc:
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    if pe not in _PE:
        raise ValueError(f"pe must be one of {list(_PE)}")
    return Desc(max_batch, n_q_heads, n_kv_heads, head_dim, prefix_max, window, _DTYPES[dtype],
                max_chunk, float(rope_base), float(scale), n_shared_prefixes, shared_prefix_max,
                _PE[pe], block_size, n_blocks)


def cache_bytes(desc: Desc) -> int:
    n = lib.psa_cache_bytes(ctypes.byref(desc))
    if n == 0:
        raise PsaError(PSA_ERR_ARG, "psa_cache_bytes")
    return n


def cache_layout(desc: Desc) -> Layout:
    out = Layout()
    _check(lib.psa_cache_layout(ctypes.byref(desc), ctypes.byref(out)), "psa_cache_layout")
    return out


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Cache:
    """A bounded prefix+window KV cache living in one torch-owned device buffer."""

    def __init__(self, max_batch: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 prefix_max: int, window: int, dtype: torch.dtype = torch.bfloat16,
                 rope_base: float = 10000.0, scale: float = 0.0, max_chunk: int = 0,
                 device=None, stream=None, n_shared_prefixes: int = 0, shared_prefix_max: int = 0,
                 pe: str = "continue", block_size: int = 0, n_blocks: int = 0):
        self.desc = make_desc(max_batch, n_q_heads, n_kv_heads, head_dim, prefix_max, window,
                              dtype, rope_base, scale, max_chunk, n_shared_prefixes,
                              shared_prefix_max, pe, block_size, n_blocks)
        self.block_size = block_size
        self.pe = pe
        self.n_shared, self.shared_max = n_shared_prefixes, shared_prefix_max
        self.dtype = dtype
        self.B, self.Hq, self.Hkv, self.D = max_batch, n_q_heads, n_kv_heads, head_dim
        self.P_max, self.W, self.max_chunk = prefix_max, window, max_chunk
        self.device = torch.device("cuda") if device is None else torch.device(device)
        self.layout = cache_layout(self.desc)
        self.nbytes = self.layout.total_bytes
        self.mem = torch.empty(self.nbytes, dtype=torch.uint8, device=self.device)
        self._h = ctypes.c_void_p()
        _check(lib.psa_cache_create(ctypes.byref(self.desc), _ptr(self.mem), self.nbytes,
                                    _stream(stream), ctypes.byref(self._h)), "psa_cache_create")

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            lib.psa_cache_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- raw device views (documented layout), for inspection -----------------------------
    def raw_tags(self) -> torch.Tensor:
        S = self.layout.slots
        return self.mem[self.layout.tags_offset:self.layout.tags_offset + self.B * S * 4] \
            .view(torch.int32).view(self.B, S)

    def raw_kv(self) -> Tuple[torch.Tensor, torch.Tensor]:
        """K and V storage: [B][H_kv][S][D], or [H_kv][n_blocks][block_size][D] when paged."""
        S, e = self.layout.slots, self.layout.elem_bytes
        if self.block_size:
            shape = (self.Hkv, self.layout.n_blocks, self.block_size, self.D)
        else:
            shape = (self.B, self.Hkv, S, self.D)
        n = shape[0] * shape[1] * shape[2] * shape[3] * e
        k = self.mem[self.layout.k_offset:self.layout.k_offset + n].view(self.dtype)
        v = self.mem[self.layout.v_offset:self.layout.v_offset + n].view(self.dtype)
        return k.view(shape), v.view(shape)

    def blocks(self, seq: int) -> Tuple[List[int], int]:
        """Paged caches: (block table of `seq`, one physical block or -1 per logical block;
        free blocks in the pool), from the host's allocator."""
        nb = self.layout.slots // self.block_size if self.block_size else 0
        table = (ctypes.c_int32 * max(nb, 1))()
        n, free = ctypes.c_int32(), ctypes.c_int32()
        _check(lib.psa_seq_blocks(self._h, seq, table, ctypes.byref(n), ctypes.byref(free)),
               "psa_seq_blocks")
        return list(table[:n.value]), free.value

    # -- calls ---------------------------------------------------------------------------
    def reset(self, seq: int, prefix_len: int, stream=None) -> None:
        _check(lib.psa_seq_reset(self._h, seq, prefix_len, _stream(stream)), "psa_seq_reset")

    def prefix_load(self, prefix_id: int, k: torch.Tensor, v: torch.Tensor, stream=None) -> None:
        """Write shared-prefix entry `prefix_id`: k, v [len][H_kv][D] at positions 0 .. len-1."""
        for name, t in (("k", k), ("v", v)):
            if t.dtype != self.dtype or not t.is_contiguous() or t.dim() != 3 or \
                    tuple(t.shape[1:]) != (self.Hkv, self.D):
                raise ValueError(f"{name} must be a contiguous {self.dtype} [len][{self.Hkv}][{self.D}] tensor")
        if k.shape[0] != v.shape[0]:
            raise ValueError("k and v differ in length")
        _check(lib.psa_prefix_load(self._h, prefix_id, k.shape[0], _ptr(k), _ptr(v), _stream(stream)),
               "psa_prefix_load")

    def attach(self, seq: int, prefix_id: int, stream=None) -> None:
        """Start sequence `seq` on shared-prefix entry `prefix_id`."""
        _check(lib.psa_seq_attach(self._h, seq, prefix_id, _stream(stream)), "psa_seq_attach")

    def set_window(self, seq: int, window: int, stream=None) -> None:
        """Window length of sequence `seq` from now on (1 .. W); a longer window drops its
        oldest entries at once."""
        _check(lib.psa_seq_set_window(self._h, seq, window, _stream(stream)), "psa_seq_set_window")

    def promote(self, seq: int, count: int, stream=None) -> None:
        """Move the `count` oldest window entries of `seq` into its pinned prefix."""
        _check(lib.psa_seq_promote(self._h, seq, count, _stream(stream)), "psa_seq_promote")

    def window_info(self, seq: int) -> Tuple[int, int, int]:
        """(window length, pinned entries, window entries) of `seq` from the host mirror."""
        w, pin, ent = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(lib.psa_seq_window(self._h, seq, ctypes.byref(w), ctypes.byref(pin),
                                  ctypes.byref(ent)), "psa_seq_window")
        return w.value, pin.value, ent.value

    def _kv_check(self, t: torch.Tensor, name: str, heads: int) -> int:
        if t.dtype != self.dtype or not t.is_contiguous() or t.device.type != "cuda":
            raise ValueError(f"{name} must be a contiguous {self.dtype} CUDA tensor")
        if t.dim() != 4 or t.shape[0] != self.B or t.shape[2] != heads or t.shape[3] != self.D:
            raise ValueError(f"{name} must be [B={self.B}][n][{heads}][{self.D}], got {tuple(t.shape)}")
        return t.shape[1]

    def append(self, k: torch.Tensor, v: torch.Tensor, n_new: Optional[Sequence[int]] = None,
               stream=None) -> None:
        """k, v: [B][n_stride][H_kv][D]; n_new: per-sequence counts (default n_stride each)."""
        n_stride = self._kv_check(k, "k", self.Hkv)
        if self._kv_check(v, "v", self.Hkv) != n_stride:
            raise ValueError("k and v differ in length")
        if n_new is None:
            arr, uni = None, n_stride
        else:
            if len(n_new) != self.B:
                raise ValueError("n_new needs one entry per sequence")
            arr, uni = (ctypes.c_int32 * self.B)(*[int(x) for x in n_new]), 0
        _check(lib.psa_append(self._h, arr, uni, _ptr(k), _ptr(v), n_stride, _stream(stream)),
               "psa_append")

    def decode(self, q: torch.Tensor, out: Optional[torch.Tensor] = None,
               lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
        """q: [B][H_q][D] for the most recently appended token of each sequence."""
        if q.dtype != self.dtype or not q.is_contiguous() or tuple(q.shape) != (self.B, self.Hq, self.D):
            raise ValueError(f"q must be a contiguous {self.dtype} [B][H_q][D] tensor")
        if out is None:
            out = torch.empty_like(q)
        if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (self.B, self.Hq)
                                or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 [B][H_q] tensor")
        _check(lib.psa_decode_attn(self._h, _ptr(q), _ptr(out), _ptr(lse), _stream(stream)),
               "psa_decode_attn")
        return out

    def decode_step(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor,
                    out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
        """Append one token per sequence (k, v: [B][H_kv][D]) and decode it (q: [B][H_q][D])
        in one launch; same result as append(k[:, None], v[:, None]) then decode(q)."""
        for name, t in (("k", k), ("v", v)):
            if t.dtype != self.dtype or not t.is_contiguous() or tuple(t.shape) != (self.B, self.Hkv, self.D):
                raise ValueError(f"{name} must be a contiguous {self.dtype} [B][H_kv][D] tensor")
        if q.dtype != self.dtype or not q.is_contiguous() or tuple(q.shape) != (self.B, self.Hq, self.D):
            raise ValueError(f"q must be a contiguous {self.dtype} [B][H_q][D] tensor")
        if out is None:
            out = torch.empty_like(q)
        if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (self.B, self.Hq)
                                or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 [B][H_q] tensor")
        _check(lib.psa_decode_step(self._h, _ptr(k), _ptr(v), _ptr(q), _ptr(out), _ptr(lse),
                                   _stream(stream)), "psa_decode_step")
        return out

    def prefill(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
        """q: [B][C][H_q][D]; k, v: [B][C][H_kv][D]. Attends, then appends the chunk."""
        C = self._kv_check(k, "k", self.Hkv)
        if self._kv_check(v, "v", self.Hkv) != C or self._kv_check(q, "q", self.Hq) != C:
            raise ValueError("q, k and v differ in chunk length")
        if out is None:
            out = torch.empty_like(q)
        if lse is not None and (lse.dtype != torch.float32 or tuple(lse.shape) != (self.B, C, self.Hq)
                                or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 [B][C][H_q] tensor")
        _check(lib.psa_prefill_attn(self._h, C, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
                                    _stream(stream)), "psa_prefill_attn")
        return out

    def export(self, seq: int, stream=None):
        """Logical view of one sequence on the host: (k [n][H_kv][D], v, positions [n])."""
        cap = max(self.P_max, self.shared_max) + self.W
        k = torch.empty((cap, self.Hkv, self.D), dtype=self.dtype)
        v = torch.empty_like(k)
        pos = torch.empty(cap, dtype=torch.int32)
        cnt = ctypes.c_int32()
        _check(lib.psa_export(self._h, seq, _ptr(k), _ptr(v), _ptr(pos), ctypes.byref(cnt),
                              _stream(stream)), "psa_export")
        n = cnt.value
        return k[:n], v[:n], pos[:n]

    def seq_length(self, seq: int) -> int:
        return lib.psa_seq_length(self._h, seq)

    def set_split_tokens(self, tokens: int) -> None:
        _check(lib.psa_set_split_tokens(self._h, tokens), "psa_set_split_tokens")

    def profile(self, enable: bool) -> None:
        _check(lib.psa_profile(self._h, 1 if enable else 0), "psa_profile")

    def profile_read(self, kernel: int) -> Tuple[float, int]:
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        _check(lib.psa_profile_read(self._h, kernel, ctypes.byref(ms), ctypes.byref(n)),
               "psa_profile_read")
        return ms.value, n.value


class TrainAttention:
    """Masked attention forward and backward on caller tensors (bf16, row space).

    q, out, dout, dq: [B][T][H_q][D]; k, v, dk, dv: [B][T][H_kv][D]; lse [B][T][H_q] float32.
    prefix[b] rows are the pinned prefix of sequence b; lens[b] its valid rows (default T).
    """

    def __init__(self, batch: int, seq_len: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 window: int, scale: float = 0.0, device="cuda"):
        self.desc = TrainDesc(batch, seq_len, n_q_heads, n_kv_heads, head_dim, window, scale, 0)
        nb = lib.psa_train_workspace_bytes(ctypes.byref(self.desc))
        if nb == 0:
            raise PsaError(PSA_ERR_ARG, "psa_train_workspace_bytes")
        self.ws = torch.empty(nb, dtype=torch.uint8, device=device)
        self.B, self.T, self.Hq, self.Hkv, self.D = batch, seq_len, n_q_heads, n_kv_heads, head_dim

    def _seq(self, prefix, lens):
        if len(prefix) != self.B or (lens is not None and len(lens) != self.B):
            raise ValueError("prefix and lens need one entry per sequence")
        pre = (ctypes.c_int32 * self.B)(*[int(x) for x in prefix])
        ln = None if lens is None else (ctypes.c_int32 * self.B)(*[int(x) for x in lens])
        return pre, ln

    def _check(self, t: torch.Tensor, name: str, heads: int, dtype=torch.bfloat16) -> None:
        want = (self.B, self.T, heads) + (() if dtype == torch.float32 else (self.D,))
        if t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != want or t.device.type != "cuda":
            raise ValueError(f"{name} must be a contiguous {dtype} CUDA tensor of shape {want}")

    def forward(self, q, k, v, prefix, lens=None, out=None, lse=None, stream=None):
        for name, t, hh in (("q", q, self.Hq), ("k", k, self.Hkv), ("v", v, self.Hkv)):
            self._check(t, name, hh)
        out = torch.empty_like(q) if out is None else out
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse is None else lse
        self._check(out, "out", self.Hq)
        self._check(lse, "lse", self.Hq, torch.float32)
        pre, ln = self._seq(prefix, lens)
        _check(lib.psa_train_fwd(ctypes.byref(self.desc), pre, ln, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(out), _ptr(lse), _ptr(self.ws), self.ws.numel(),
                                 _stream(stream)), "psa_train_fwd")
        return out, lse

    def backward(self, q, k, v, out, lse, dout, prefix, lens=None, dq=None, dk=None, dv=None,
                 stream=None):
        for name, t, hh in (("q", q, self.Hq), ("k", k, self.Hkv), ("v", v, self.Hkv),
                            ("out", out, self.Hq), ("dout", dout, self.Hq)):
            self._check(t, name, hh)
        self._check(lse, "lse", self.Hq, torch.float32)
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        pre, ln = self._seq(prefix, lens)
        _check(lib.psa_train_bwd(ctypes.byref(self.desc), pre, ln, _ptr(q), _ptr(k), _ptr(v),
                                 _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                 _ptr(self.ws), self.ws.numel(), _stream(stream)), "psa_train_bwd")
        return dq, dk, dv

    def backward_noalloc(self, q, k, v, out, lse, dout, prefix, lens=None, dq=None, dk=None,
                         dv=None, stream=None):
        """backward() through psa_train_bwd_noalloc: the library's static scratch instead of
        this object's workspace (the outputs must be given to allocate nothing here)."""
        for name, t, hh in (("q", q, self.Hq), ("k", k, self.Hkv), ("v", v, self.Hkv),
                            ("out", out, self.Hq), ("dout", dout, self.Hq)):
            self._check(t, name, hh)
        self._check(lse, "lse", self.Hq, torch.float32)
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        for name, t, hh in (("dq", dq, self.Hq), ("dk", dk, self.Hkv), ("dv", dv, self.Hkv)):
            self._check(t, name, hh)
        pre, ln = self._seq(prefix, lens)
        _check(lib.psa_train_bwd_noalloc(ctypes.byref(self.desc), pre, ln, _ptr(q), _ptr(k),
                                         _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _ptr(dq),
                                         _ptr(dk), _ptr(dv), _stream(stream)),
               "psa_train_bwd_noalloc")
        return dq, dk, dv
