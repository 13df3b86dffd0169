"""Chunked prefill on the GPU against the float64 oracle.

A chunk of C tokens at positions n .. n + C - 1: row c must equal the oracle's attention of
the query at p = n + c over A(p) (the chunk being C consecutive decode steps), and after the
call the cache must hold the chunk exactly as C single appends would (bit for bit).
Tolerances as for decode: max-abs <= 2e-2 and rel-L2 <= 5e-3 (bf16), lse within 2e-2."""
import numpy as np
import pytest
import torch

from oracle import attn, cache as ocache
from synth import configs, drive

pytestmark = pytest.mark.gpu


def bits(t):
    return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def tol_check(out, ref, what=""):
    err = np.abs(out - ref).max()
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    assert err <= 2e-2 and rel <= 5e-3, f"{what} max-abs {err} rel-l2 {rel}"
    return err, rel


def run_chunk(c, wl, n_before, C, rows=None, seqs=None, check_cache=True):
    B = wl.batch
    q = drive.query_block(wl, n_before, C, "cuda")
    k, v = drive.kv_block(wl, n_before, C, "cuda")
    lse = torch.empty((B, C, wl.n_q_heads), dtype=torch.float32, device="cuda")
    out = c.prefill(q, k, v, lse=lse)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    assert np.isfinite(o).all()
    qc = q.double().cpu().numpy()
    lc = lse.cpu().numpy()
    seqs = range(B) if seqs is None else seqs
    rows_ = list(range(C)) if rows is None else rows
    outs, refs = [], []
    for b in seqs:
        ref, ref_lse = attn.prefill_chunk(qc[b], n_before[b], drive.hist_provider(wl, b),
                                          wl.prefix[b], wl.window, wl.n_kv_heads, wl.rope_base,
                                          wl.scale, rows=rows_)
        outs.append(o[b][rows_])
        refs.append(ref)
        np.testing.assert_allclose(lc[b][rows_], ref_lse, rtol=0, atol=2e-2)
        if check_cache:
            n = n_before[b] + C
            assert c.seq_length(b) == n
            k_e, v_e, pos_e = c.export(b)
            pos, kbits, vref = ocache.expected_view(wl.prefix[b], wl.window, n,
                                                    drive.hist_provider(wl, b), wl.rope_base, "bf16")
            assert pos_e.tolist() == pos.tolist()
            np.testing.assert_array_equal(bits(k_e), kbits)
            np.testing.assert_array_equal(v_e.double().numpy(), vref)
    return tol_check(np.stack(outs), np.stack(refs))


SHAPES = [(128, 16, 8), (128, 8, 8), (128, 32, 8), (128, 64, 8), (64, 16, 8), (64, 8, 4)]


@pytest.mark.parametrize("D,Hq,Hkv", SHAPES)
def test_phases(D, Hq, Hkv):
    # sequences: empty cache, chunk crossing the end of the prefix, window still filling,
    # window full, chunk longer than the window is irrelevant here (C = 100 < W = 150)
    W, C = 150, 100
    prefix = [20, 60, 10, 30, 0]
    n_hist = [0, 40, 90, 700, 333]
    wl = configs.Workload("pf", torch.bfloat16, 5, Hq, Hkv, D, W, prefix, [1] * 5, "prefill")
    c = drive.make_cache(wl, max_chunk=C)
    drive.fill(c, wl, n_hist)
    run_chunk(c, wl, n_hist, C)


def test_chunk_longer_than_window():
    # C > W: later rows no longer see the chunk's first tokens; tokens the chunk itself
    # evicts are never written to the cache.
    W, C = 48, 200
    prefix = [5, 0, 17]
    n_hist = [0, 100, 30]
    wl = configs.Workload("pf-long", torch.bfloat16, 3, 16, 8, 128, W, prefix, [1] * 3, "prefill")
    c = drive.make_cache(wl, max_chunk=C)
    drive.fill(c, wl, n_hist)
    run_chunk(c, wl, n_hist, C)


def test_consecutive_chunks_then_decode():
    W, C = 200, 96
    prefix = [50, 13]
    wl = configs.Workload("pf-seq", torch.bfloat16, 2, 16, 8, 128, W, prefix, [1, 1], "prefill")
    c = drive.make_cache(wl, max_chunk=C)
    for b in range(2):
        c.reset(b, prefix[b])
    n = [0, 0]
    for _ in range(5):                       # 480 tokens: prefix, filling, full, evicting
        run_chunk(c, wl, n, C)
        n = [x + C for x in n]
    # a decode step on top of the prefilled cache
    k, v = drive.kv_block(wl, n, 1, "cuda")
    c.append(k, v)
    q = drive.queries(wl, n, "cuda")
    out = c.decode(q).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(2):
        ref, _ = attn.decode_query(qc[b], n[b], drive.hist_provider(wl, b), prefix[b], W,
                                   wl.n_kv_heads, wl.rope_base, wl.scale)
        tol_check(out[b], ref, f"decode after prefill seq {b}")


def test_single_token_chunk_equals_decode():
    W = 64
    wl = configs.Workload("pf-one", torch.bfloat16, 2, 16, 8, 128, W, [10, 0], [1, 1], "prefill")
    c = drive.make_cache(wl, max_chunk=8)
    drive.fill(c, wl, [300, 5])
    run_chunk(c, wl, [300, 5], 1)


def test_float32_storage_rejected():
    import prefix_pinned_sliding_amd as psa
    wl = configs.Workload("pf-f32", torch.float32, 1, 4, 4, 64, 8, [2], [1], "prefill")
    c = drive.make_cache(wl, max_chunk=4)
    c.reset(0, 2)
    q = torch.zeros((1, 4, 4, 64), device="cuda")
    k = torch.zeros((1, 4, 4, 64), device="cuda")
    with pytest.raises(psa.PsaError) as e:
        c.prefill(q, k, k.clone())
    assert e.value.status == psa.PSA_ERR_ARG
    assert c.seq_length(0) == 0


def test_prefill_chunk512_full_size():
    wl = configs.prefill_chunk512()
    n_hist = [t - 1 for t in wl.start]
    c = drive.make_cache(wl, max_chunk=wl.chunk)
    drive.fill(c, wl, n_hist)
    rows = [0, 1, 2, 63, 64, 127, 200, 255, 256, 400, 510, 511]
    err, rel = run_chunk(c, wl, n_hist, wl.chunk, rows=rows, seqs=[0, 3, 7], check_cache=True)
    print(f"{wl.name}: max-abs {err:.2e} rel-l2 {rel:.2e}")
