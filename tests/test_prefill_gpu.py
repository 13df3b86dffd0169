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


@pytest.mark.parametrize("factor", [16.0, 64.0, -32.0])
def test_large_logits(factor):
    # Queries scaled by a power of two (exact in bf16): logits in the log2 domain reach far
    # past +-64, so the softmax reference leaves 0 (a row's first visible tile takes its
    # maximum, later tiles move it up and rescale O and l). Every value row of a sequence is
    # the same vector, so each output row must equal it exactly whatever the weights (O and
    # l rescaled alike), and lse must match the oracle within the key-rounding bound, which
    # grows with |factor|.
    W, C = 300, 128
    prefix = [40, 0, 7]
    n_hist = [900, 250, 20]
    B, Hkv, D = 3, 8, 128
    wl = configs.Workload("pf-big", torch.bfloat16, B, 16, Hkv, D, W, prefix, [1] * B, "prefill")
    c = drive.make_cache(wl, max_chunk=C)
    for b in range(B):
        c.reset(b, prefix[b])
    T = max(n_hist) + C
    k_all, _ = drive.kv_block(wl, [0] * B, T, "cuda")
    vrow = (torch.arange(B * Hkv * D, device="cuda").view(B, 1, Hkv, D) % 17 - 8).to(torch.bfloat16) / 4
    v_all = vrow.expand(B, T, Hkv, D).contiguous()
    c.append(k_all[:, :max(n_hist)].contiguous(), v_all[:, :max(n_hist)].contiguous(), n_new=n_hist)
    q = drive.query_block(wl, n_hist, C, "cuda") * factor
    kc = torch.stack([k_all[b, n_hist[b]:n_hist[b] + C] for b in range(B)]).contiguous()
    vc = v_all[:, :C].contiguous()
    lse = torch.empty((B, C, wl.n_q_heads), dtype=torch.float32, device="cuda")
    out = c.prefill(q, kc, vc, lse=lse)
    torch.cuda.synchronize()
    want = vrow[:, 0].repeat_interleave(wl.n_q_heads // Hkv, dim=1)        # [B][Hq][D]
    assert torch.equal(out, want.unsqueeze(1).expand_as(out)), "outputs differ from the constant value row"
    lc, qc = lse.cpu().numpy(), q.double().cpu().numpy()
    kd, vd = k_all.double().cpu().numpy(), v_all.double().cpu().numpy()
    for b in range(B):
        hist = attn.array_history(kd[b], vd[b])
        _, ref_lse = attn.prefill_chunk(qc[b], n_hist[b], hist, prefix[b], W, Hkv, wl.rope_base,
                                        wl.scale)
        np.testing.assert_allclose(lc[b], ref_lse, rtol=0, atol=2e-2 * abs(factor))


def test_first_keys_far_below_zero():
    # Every logit is about -261 in the log2 domain: keys carry all their energy in the
    # lowest-frequency rotation pair (dims D/2 - 1 and D - 1, turned by less than 0.04 rad over
    # these positions) and queries point the other way. A row's first visible tile then takes
    # its maximum as the softmax reference while O and l are still zero; forming the rescale
    # factor 2^261 there would overflow and turn them into NaN. The logits of a row differ by
    # less than 0.1 (log2) from key to key, about what rounding the rotated keys to bf16 moves
    # them, so the weights are not compared: every value row of a sequence is the same
    # vector, and each output row must equal it exactly. lse against the oracle within the
    # rounding of the two nonzero components of the rotated, scaled query (|q_i| < 17, bf16
    # error <= 1/16) and of the rotated key (|k_i| < 8.5, error <= 1/32):
    # 2 (8.5 / 16 + 17 / 32) = 2.1 in log2, 1.47 in natural log.
    W, C = 64, 96
    prefix = [5, 0]
    n_hist = [150, 40]
    B, Hkv, Hq, D = 2, 8, 16, 128
    wl = configs.Workload("pf-neg", torch.bfloat16, B, Hq, Hkv, D, W, prefix, [1] * B, "prefill")
    c = drive.make_cache(wl, max_chunk=C)
    for b in range(B):
        c.reset(b, prefix[b])
    T = max(n_hist) + C
    u = torch.zeros(D)
    u[D // 2 - 1] = 8.0
    u[D - 1] = 8.0
    k_all = u.to(torch.bfloat16).view(1, 1, 1, D).expand(B, T, Hkv, D).contiguous().cuda()
    vrow = (torch.arange(B * Hkv * D, device="cuda").view(B, 1, Hkv, D) % 13 - 6).to(torch.bfloat16) / 8
    v_all = vrow.expand(B, T, Hkv, D).contiguous()
    c.append(k_all[:, :max(n_hist)].contiguous(), v_all[:, :max(n_hist)].contiguous(), n_new=n_hist)
    q = (-16.0 * u).to(torch.bfloat16).view(1, 1, 1, D).expand(B, C, Hq, D).contiguous().cuda()
    kc = torch.stack([k_all[b, n_hist[b]:n_hist[b] + C] for b in range(B)]).contiguous()
    vc = v_all[:, :C].contiguous()
    lse = torch.empty((B, C, Hq), dtype=torch.float32, device="cuda")
    out = c.prefill(q, kc, vc, lse=lse)
    torch.cuda.synchronize()
    want = vrow[:, 0].repeat_interleave(Hq // Hkv, dim=1)        # [B][Hq][D]
    assert torch.equal(out, want.unsqueeze(1).expand_as(out)), "outputs differ from the constant value row"
    lc = lse.cpu().numpy()
    kd, vd, qd = k_all.double().cpu().numpy(), v_all.double().cpu().numpy(), q.double().cpu().numpy()
    for b in range(B):
        _, ref_lse = attn.prefill_chunk(qd[b], n_hist[b], attn.array_history(kd[b], vd[b]),
                                        prefix[b], W, Hkv, wl.rope_base, wl.scale)
        assert ref_lse.max() < -128 * np.log(2), "the workload must reach past the overflow"
        np.testing.assert_allclose(lc[b], ref_lse, rtol=0, atol=1.47)


def test_window_of_one_chunks():
    # W = 1 with chunks: row c sees the prefix and itself; P = 0 gives the value rows exactly
    W, C = 1, 40
    prefix = [0, 6]
    wl = configs.Workload("pf-w1", torch.bfloat16, 2, 16, 8, 128, W, prefix, [1, 1], "prefill")
    c = drive.make_cache(wl, max_chunk=C)
    for b in range(2):
        c.reset(b, prefix[b])
    n = [0, 0]
    for _ in range(3):
        q = drive.query_block(wl, n, C, "cuda")
        k, v = drive.kv_block(wl, n, C, "cuda")
        out = c.prefill(q, k, v)
        assert torch.equal(out[0], v[0].repeat_interleave(2, dim=1))
        n = [x + C for x in n]
    n = [0, 0]
    c2 = drive.make_cache(wl, max_chunk=C)
    for b in range(2):
        c2.reset(b, prefix[b])
    run_chunk(c2, wl, n, C)
