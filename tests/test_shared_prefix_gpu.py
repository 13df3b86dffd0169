"""Shared pinned prefixes ([KV-Lean] 6.1-6.2; [PS] 07: many runs of one prompt).

A sequence attached to a pool entry must behave exactly like a sequence that appended the
same prefix itself: bit-identical decode outputs and stored bytes for identical histories,
and parity with the float64 oracle (whose history for an attached sequence is the pool
prefix followed by the sequence's own tokens)."""
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


def setup(P=37, W=64, n_window=150, G=2, shared_only=False):
    # seq 0: private prefix (values of seq 0), window of seq 0
    # seq 1: private prefix (values of seq 0), window of seq 1
    # seq 2: attached to pool entry 0 (values of seq 0), window of seq 0  == seq 0's history
    # seq 3: attached to pool entry 0, window of seq 1                   == seq 1's history
    Hkv = 4
    wl = configs.Workload("shared", torch.bfloat16, 4, Hkv * G, Hkv, 128, W, [P] * 4, [1] * 4,
                          "decode")
    c = drive.make_cache(wl, max_chunk=64, n_shared=2, shared_max=P + 5)
    kp, vp = drive.kv_rows_from(wl, [0], [0], P, "cuda")
    c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())
    c.reset(0, P)
    c.reset(1, P)
    c.attach(2, 0)
    c.attach(3, 0)
    # private sequences append the prefix themselves (seq 0's values)
    k, v = drive.kv_rows_from(wl, [0, 0, 0, 0], [0] * 4, P, "cuda")
    c.append(k, v, n_new=[P, P, 0, 0])
    assert [c.seq_length(b) for b in range(4)] == [P] * 4
    src = [0, 1, 0, 1]
    k, v = drive.kv_rows_from(wl, src, [P] * 4, n_window, "cuda")
    c.append(k, v)
    return wl, c, src, P + n_window


def test_attached_matches_private_bit_for_bit_and_oracle():
    wl, c, src, n = setup()
    P = wl.prefix[0]
    k, v = drive.kv_rows_from(wl, src, [n] * 4, 1, "cuda")
    c.append(k, v)
    q = drive.queries(wl, [n] * 4, "cuda", seqs=src)
    lse = torch.empty((4, wl.n_q_heads), dtype=torch.float32, device="cuda")
    out = c.decode(q, lse=lse)
    torch.cuda.synchronize()
    assert torch.equal(out[2], out[0]) and torch.equal(out[3], out[1])
    assert torch.equal(lse[2], lse[0]) and torch.equal(lse[3], lse[1])
    qc = q.double().cpu().numpy()
    o = out.double().cpu().numpy()
    for b in range(4):
        hist = drive.composite_history(wl, 0, src[b], P)
        ref, _ = attn.decode_query(qc[b], n, hist, P, wl.window, wl.n_kv_heads, wl.rope_base,
                                   wl.scale)
        tol_check(o[b], ref, f"seq {b}")
        k_e, v_e, pos_e = c.export(b)
        pos, kbits, vref = ocache.expected_view(P, wl.window, n + 1, hist, wl.rope_base, "bf16")
        assert pos_e.tolist() == pos.tolist()
        np.testing.assert_array_equal(bits(k_e), kbits)
        np.testing.assert_array_equal(v_e.double().numpy(), vref)


def test_attached_prefill_matches_private():
    wl, c, src, n = setup(n_window=40)
    P = wl.prefix[0]
    C = 48
    q = torch.stack([drive.query_block(wl, [n] * 4, C, "cuda")[s] for s in src]).contiguous()
    k, v = drive.kv_rows_from(wl, src, [n] * 4, C, "cuda")
    out = c.prefill(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out[2], out[0]) and torch.equal(out[3], out[1])
    qc = q.double().cpu().numpy()
    o = out.double().cpu().numpy()
    for b in (1, 3):
        hist = drive.composite_history(wl, 0, src[b], P)
        ref, _ = attn.prefill_chunk(qc[b], n, hist, P, wl.window, wl.n_kv_heads, wl.rope_base,
                                    wl.scale)
        tol_check(o[b], ref, f"prefill seq {b}")


def test_prefix_longer_than_private_slots():
    # a cache with no private prefix slots at all: every prompt lives in the pool
    W, P = 32, 50
    wl = configs.Workload("pool-only", torch.bfloat16, 2, 16, 8, 128, W, [P, 20], [1, 1], "decode")
    c = drive.make_cache(wl, n_shared=2, shared_max=64, prefix_max=0)
    for e, (src, L) in enumerate([(0, P), (1, 20)]):
        kp, vp = drive.kv_rows_from(wl, [src], [0], L, "cuda")
        c.prefix_load(e, kp[0].contiguous(), vp[0].contiguous())
        c.attach(e, e)
    k, v = drive.kv_rows_from(wl, [0, 1], [P, 20], 70, "cuda")
    c.append(k, v)
    n = [P + 70, 20 + 70]
    k, v = drive.kv_rows_from(wl, [0, 1], n, 1, "cuda")
    c.append(k, v)
    q = drive.queries(wl, n, "cuda")
    out = c.decode(q).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(2):
        ref, _ = attn.decode_query(qc[b], n[b], drive.hist_provider(wl, b), wl.prefix[b], W,
                                   wl.n_kv_heads, wl.rope_base, wl.scale)
        tol_check(out[b], ref, f"seq {b}")
        k_e, _, pos_e = c.export(b)
        pos, kbits, _ = ocache.expected_view(wl.prefix[b], W, n[b] + 1,
                                             drive.hist_provider(wl, b), wl.rope_base, "bf16")
        assert pos_e.tolist() == pos.tolist()
        np.testing.assert_array_equal(bits(k_e), kbits)


def test_pool_state_errors():
    import prefix_pinned_sliding_amd as psa
    wl = configs.Workload("err", torch.bfloat16, 2, 8, 4, 64, 16, [4, 4], [1, 1], "decode")
    c = drive.make_cache(wl, n_shared=1, shared_max=8)
    kp, vp = drive.kv_rows_from(wl, [0], [0], 6, "cuda")
    with pytest.raises(psa.PsaError) as e:
        c.attach(0, 0)                       # never loaded
    assert e.value.status == psa.PSA_ERR_STATE
    with pytest.raises(psa.PsaError) as e:
        c.attach(0, 1)                       # out of range
    assert e.value.status == psa.PSA_ERR_ARG
    kl, vl = drive.kv_rows_from(wl, [0], [0], 9, "cuda")
    with pytest.raises(psa.PsaError) as e:
        c.prefix_load(0, kl[0].contiguous(), vl[0].contiguous())   # longer than shared_max
    assert e.value.status == psa.PSA_ERR_ARG
    c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())
    c.attach(0, 0)
    assert c.seq_length(0) == 6
    with pytest.raises(psa.PsaError) as e:
        c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())   # entry in use
    assert e.value.status == psa.PSA_ERR_STATE
    c.reset(0, 2)                            # detaches
    c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())


@pytest.mark.parametrize("fused", [False, True])
def test_long_shared_prefix_over_a_short_private_prefix(fused):
    # prefix_max = 0 and a pool entry of 512 tokens with W = 128: an attached sequence sees
    # 640 entries, five splits of 128, more than prefix_max + W alone would give room for.
    # Each split's partial result needs its own workspace slot (a regression test of the
    # workspace sizing), checked against the oracle at 128-entry splits and automatic ones.
    P, W, B, Hkv, G = 512, 128, 3, 2, 4
    wl = configs.Workload("shared-long", torch.bfloat16, B, Hkv * G, Hkv, 128, W, [P] * B,
                          [1] * B, "decode")
    c = drive.make_cache(wl, n_shared=1, shared_max=P, prefix_max=0)
    kp, vp = drive.kv_rows_from(wl, [0], [0], P, "cuda")
    c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())
    for b in range(B):
        c.attach(b, 0)
    n_win = [300, 5, 128]
    k, v = drive.kv_rows_from(wl, list(range(B)), [P] * B, max(n_win), "cuda")
    c.append(k, v, n_new=n_win)
    n = [P + x for x in n_win]
    for tokens in (128, 0):
        c.set_split_tokens(tokens)
        k, v = drive.kv_rows_from(wl, list(range(B)), n, 1, "cuda")
        q = drive.queries(wl, n, "cuda")
        if fused:
            out = c.decode_step(k[:, 0].contiguous(), v[:, 0].contiguous(), q)
        else:
            c.append(k, v)
            out = c.decode(q)
        torch.cuda.synchronize()
        o = out.double().cpu().numpy()
        qc = q.double().cpu().numpy()
        for b in range(B):
            hist = drive.composite_history(wl, 0, b, P)
            ref, _ = attn.decode_query(qc[b], n[b], hist, P, W, Hkv, wl.rope_base, wl.scale)
            tol_check(o[b], ref, f"split {tokens} seq {b}")
        n = [x + 1 for x in n]
