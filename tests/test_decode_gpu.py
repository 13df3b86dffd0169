"""Decode attention on the GPU against the float64 oracle (masked full history).

Tolerances: max|out - ref| <= 1e-5 for float32; for bfloat16, max-abs <= 2e-2 and
||out - ref||_2 / ||ref||_2 <= 5e-3 over each call's checked outputs.

lse: the oracle rotates keys in float64 without rounding, the cache holds them rounded
once to the storage type, so each logit carries an error of at most
scale * sum_d |q_d| |k_d| * 2^-8 (half an ulp, relative 2^-8 at worst). For N(0,1)
inputs at D = 128 that bound is about 0.03 for bfloat16 (typical errors ~1e-3) and
about 1e-6 for float32 storage (2^-24). lse is a weighted mean of logits plus a log,
so it inherits the same bound: checked at 2e-2 (bfloat16) and 1e-5 (float32). The full-size
workloads are checked whole-tensor in test_full_size_gpu.py; every output here is checked to
be finite."""
import numpy as np
import pytest
import torch

from oracle import attn
from synth import configs, drive

pytestmark = pytest.mark.gpu


def tol_check(out: np.ndarray, ref: np.ndarray, dtype, what=""):
    err = np.abs(out - ref).max()
    if dtype == torch.float32:
        assert err <= 1e-5, f"{what} max-abs {err}"
    else:
        rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
        assert err <= 2e-2 and rel <= 5e-3, f"{what} max-abs {err} rel-l2 {rel}"
    return err


def oracle_decode(wl, b, p, q_row):
    return attn.decode_query(q_row, p, drive.hist_provider(wl, b), wl.prefix[b], wl.window_of(b),
                             wl.n_kv_heads, wl.rope_base, wl.scale)


def lse_tol(dtype):
    return 1e-5 if dtype == torch.float32 else 2e-2


def step_and_check(c, wl, n_before, seqs=None, lse=True):
    """Append the token at p = n_before[b], decode it, compare chosen sequences."""
    B = wl.batch
    k, v = drive.kv_block(wl, n_before, 1, "cuda")
    c.append(k, v)
    q = drive.queries(wl, n_before, "cuda")
    lse_t = torch.empty((B, wl.n_q_heads), dtype=torch.float32, device="cuda") if lse else None
    out = c.decode(q, lse=lse_t)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    assert np.isfinite(o).all()
    qc = q.double().cpu().numpy()
    seqs = range(B) if seqs is None else seqs
    outs, refs = [], []
    for b in seqs:
        ref, ref_lse = oracle_decode(wl, b, n_before[b], qc[b])
        outs.append(o[b])
        refs.append(ref)
        if lse:
            np.testing.assert_allclose(lse_t[b].cpu().numpy(), ref_lse, rtol=0, atol=lse_tol(wl.dtype))
    return np.stack(outs), np.stack(refs)


def test_tiny_fp32_all_steps():
    wl = configs.tiny_fp32()
    c = drive.make_cache(wl)
    c.reset(0, wl.prefix[0])
    worst = 0.0
    for p in range(wl.steps):
        o, r = step_and_check(c, wl, [p])
        worst = max(worst, tol_check(o, r, wl.dtype, f"step {p}"))
    print(f"tiny fp32: 200 steps, worst max-abs {worst:.2e}")


def test_first_token_returns_its_value():
    wl = configs.Workload("first", torch.bfloat16, 2, 8, 4, 128, 8, [3, 0], [1, 1], "decode")
    c = drive.make_cache(wl)
    for b in range(2):
        c.reset(b, wl.prefix[b])
    k, v = drive.kv_block(wl, [0, 0], 1, "cuda")
    c.append(k, v)
    out = c.decode(drive.queries(wl, [0, 0], "cuda"))
    G = 2
    want = v[:, 0].repeat_interleave(G, dim=1)
    assert torch.equal(out, want)


GRID = [(torch.bfloat16, 128, 16, 8), (torch.bfloat16, 128, 32, 8), (torch.bfloat16, 64, 8, 8),
        (torch.bfloat16, 128, 64, 8), (torch.float32, 64, 8, 4), (torch.float32, 128, 16, 8),
        (torch.bfloat16, 64, 32, 4)]


@pytest.mark.parametrize("dtype,D,Hq,Hkv", GRID)
def test_phases_and_shapes(dtype, D, Hq, Hkv):
    # Sequences in every phase: inside the prefix, window filling, exactly full, first
    # eviction, long after; plus P = 0 (plain sliding window).
    W = 37
    prefix = [7, 3, 20, 0, 5, 12]
    n_hist = [3, 15, 20 + W - 1, 40, 5 + W, 900]
    wl = configs.Workload("grid", dtype, len(prefix), Hq, Hkv, D, W, prefix, [1] * 6, "decode")
    c = drive.make_cache(wl)
    drive.fill(c, wl, n_hist)
    o, r = step_and_check(c, wl, n_hist)
    tol_check(o, r, dtype)


def test_split_count_invariance():
    W = 1000
    prefix = [100, 0, 37, 200]
    n_hist = [5000, 1200, 700, 250]
    wl = configs.Workload("splits", torch.bfloat16, 4, 16, 8, 128, W, prefix, [1] * 4, "decode")
    c = drive.make_cache(wl)
    drive.fill(c, wl, n_hist)
    k, v = drive.kv_block(wl, n_hist, 1, "cuda")
    c.append(k, v)
    q = drive.queries(wl, n_hist, "cuda")
    qc = q.double().cpu().numpy()
    refs = [oracle_decode(wl, b, n_hist[b], qc[b]) for b in range(4)]
    lses = []
    for tokens in (128, 256, 384, 1152, 0):
        c.set_split_tokens(tokens)
        lse = torch.empty((4, 16), dtype=torch.float32, device="cuda")
        out = c.decode(q, lse=lse).double().cpu().numpy()
        for b in range(4):
            tol_check(out[b], refs[b][0], wl.dtype, f"split {tokens} seq {b}")
        lses.append(lse.cpu().numpy())
    for x in lses[1:]:
        np.testing.assert_allclose(x, lses[0], rtol=0, atol=2e-5)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_window_of_one(dtype):
    # W = 1: each query sees its pinned prefix and itself only; with P = 0 the output is the
    # token's own value row exactly (a softmax over one key). Every step from the empty cache
    # through the prefix and well past it, on the two-call path and the fused step.
    W = 1
    prefix = [0, 3, 5]
    wl = configs.Workload("w1", dtype, 3, 8, 4, 64, W, prefix, [1] * 3, "decode")
    caches = [drive.make_cache(wl) for _ in range(2)]
    for c in caches:
        for b in range(3):
            c.reset(b, prefix[b])
    for p in range(12):
        k, v = drive.kv_block(wl, [p] * 3, 1, "cuda")
        q = drive.queries(wl, [p] * 3, "cuda")
        caches[0].append(k, v)
        o2 = caches[0].decode(q)
        of = caches[1].decode_step(k[:, 0].contiguous(), v[:, 0].contiguous(), q)
        assert torch.equal(o2, of), f"step {p}"
        assert torch.equal(o2[0], v[0, 0].repeat_interleave(2, dim=0)), f"P = 0, step {p}"
        o, qc = o2.double().cpu().numpy(), q.double().cpu().numpy()
        for b in range(3):
            ref, _ = oracle_decode(wl, b, p, qc[b])
            tol_check(o[b], ref, dtype, f"step {p} seq {b}")
