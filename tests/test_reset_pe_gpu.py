"""Reset PE ([PS] 05) on the GPU against the float64 oracle's literal renumbering."""
import numpy as np
import pytest
import torch

from oracle import attn
from synth import configs, drive

pytestmark = pytest.mark.gpu


def tol_check(out, ref, dtype, what=""):
    err = np.abs(out - ref).max()
    if dtype == torch.float32:
        assert err <= 1e-5, f"{what} max-abs {err}"
    else:
        rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
        assert err <= 2e-2 and rel <= 5e-3, f"{what} max-abs {err} rel-l2 {rel}"


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 16, 8), (torch.bfloat16, 128, 32, 8),
                                            (torch.float32, 64, 8, 4), (torch.bfloat16, 64, 8, 8)])
@pytest.mark.parametrize("split", [0, 128])
def test_decode_reset_phases(dtype, D, Hq, Hkv, split):
    W = 150
    prefix = [300, 3, 20, 0, 5, 140]
    n_hist = [40, 15, 20 + W - 1, 400, 5 + W, 2000]
    wl = configs.Workload("reset", dtype, len(prefix), Hq, Hkv, D, W, prefix, [1] * 6, "decode")
    c = drive.make_cache(wl, pe="reset")
    c.set_split_tokens(split)
    drive.fill(c, wl, n_hist)
    k, v = drive.kv_block(wl, n_hist, 1, "cuda")
    c.append(k, v)
    q = drive.queries(wl, n_hist, "cuda")
    lse = torch.empty((6, Hq), dtype=torch.float32, device="cuda")
    out = c.decode(q, lse=lse).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(6):
        ref, rl = attn.decode_query(qc[b], n_hist[b], drive.hist_provider(wl, b), prefix[b], W,
                                    Hkv, wl.rope_base, wl.scale, pe="reset")
        tol_check(out[b], ref, dtype, f"seq {b}")
        np.testing.assert_allclose(lse[b].cpu().numpy(), rl, rtol=0,
                                   atol=1e-5 if dtype == torch.float32 else 2e-2)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 16, 8), (64, 32, 8), (128, 4, 4)])
def test_prefill_reset(D, Hq, Hkv):
    """Queries are rotated in the attention kernel: first at the renumbered position for
    the prefix tiles, then again at p; both head dims and several group sizes."""
    W, C = 96, 128
    prefix = [40, 10, 0, 200]
    n_hist = [20, 300, 250, 260]
    wl = configs.Workload("reset-pf", torch.bfloat16, 4, Hq, Hkv, D, W, prefix, [1] * 4, "prefill")
    c = drive.make_cache(wl, max_chunk=C, pe="reset")
    drive.fill(c, wl, n_hist)
    q = drive.query_block(wl, n_hist, C, "cuda")
    k, v = drive.kv_block(wl, n_hist, C, "cuda")
    out = c.prefill(q, k, v).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(4):
        ref, _ = attn.prefill_chunk(qc[b], n_hist[b], drive.hist_provider(wl, b), prefix[b], W,
                                    wl.n_kv_heads, wl.rope_base, wl.scale, pe="reset")
        tol_check(out[b], ref, torch.bfloat16, f"prefill seq {b}")


def test_reset_with_shared_prefix():
    W, P = 64, 90
    wl = configs.Workload("reset-shared", torch.bfloat16, 2, 16, 8, 128, W, [P, P], [1, 1], "decode")
    c = drive.make_cache(wl, n_shared=1, shared_max=P, prefix_max=0, pe="reset")
    kp, vp = drive.kv_rows_from(wl, [0], [0], P, "cuda")
    c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())
    c.attach(0, 0)
    c.attach(1, 0)
    n = P + 500
    k, v = drive.kv_rows_from(wl, [0, 1], [P, P], 501, "cuda")
    c.append(k, v)
    q = drive.queries(wl, [n, n], "cuda")
    out = c.decode(q).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(2):
        hist = drive.composite_history(wl, 0, b, P)
        ref, _ = attn.decode_query(qc[b], n, hist, P, W, wl.n_kv_heads, wl.rope_base, wl.scale,
                                   pe="reset")
        tol_check(out[b], ref, torch.bfloat16, f"seq {b}")
