"""Pins of oracle.attn: full attention before the window fills (library SDPA in float64),
exact special cases, plain sliding window at P = 0 (the Lean article's model), agreement
of the mask form with the cache form, and leak detection."""
import numpy as np
import pytest
import torch

from oracle import attn, rope, spec


def rand_hist(rng, n, Hkv, D):
    return rng.standard_normal((n, Hkv, D)), rng.standard_normal((n, Hkv, D))


def sdpa_reference(q, p, k, v, base, scale, n_kv_heads):
    """torch scaled_dot_product_attention (float64, CPU) over keys 0..p with no mask."""
    Hq, D = q.shape
    G = Hq // n_kv_heads
    pos = np.arange(p + 1)
    qr = torch.from_numpy(rope.rotate(q, np.full(Hq, p), base))
    kr = torch.from_numpy(rope.rotate(k[: p + 1], np.broadcast_to(pos[:, None], (p + 1, n_kv_heads)), base))
    vv = torch.from_numpy(np.asarray(v[: p + 1]))
    out = np.empty((Hq, D))
    for hq in range(Hq):
        hk = hq // G
        o = torch.nn.functional.scaled_dot_product_attention(
            qr[hq].view(1, 1, 1, D), kr[:, hk].reshape(1, 1, p + 1, D).contiguous(),
            vv[:, hk].reshape(1, 1, p + 1, D).contiguous(), scale=scale)
        out[hq] = o.view(D).numpy()
    return out


@pytest.mark.parametrize("P,W,n", [(16, 32, 1), (16, 32, 10), (16, 32, 48), (0, 8, 8), (5, 3, 8),
                                   (100, 4096, 300)])
def test_full_attention_before_window_fills(P, W, n):
    # [PS] 04: until the window is full the method is plain causal attention.
    assert n <= P + W
    rng = np.random.default_rng(n)
    Hq, Hkv, D = 4, 2, 64
    k, v = rand_hist(rng, n, Hkv, D)
    q = rng.standard_normal((Hq, D))
    out, _ = attn.decode_query(q, n - 1, attn.array_history(k, v), P, W, Hkv, 10000.0, D ** -0.5)
    ref = sdpa_reference(q, n - 1, k, v, 10000.0, D ** -0.5, Hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_mask_form_equals_cache_form():
    # [KV-Lean] 4.2 corollary: attention over the bounded cache equals masked full-history attention.
    rng = np.random.default_rng(7)
    Hq, Hkv, D = 4, 2, 16
    for P in range(0, 4):
        for W in range(1, 5):
            n_max = 3 * W + P + 3
            k, v = rand_hist(rng, n_max, Hkv, D)
            h = attn.array_history(k, v)
            for p in range(n_max):
                q = rng.standard_normal((Hq, D))
                a = attn.decode_query(q, p, h, P, W, Hkv, 10000.0, 0.25)
                b = attn.decode_query_from_cache(q, p, h, P, W, Hkv, 10000.0, 0.25)
                np.testing.assert_allclose(a[0], b[0], rtol=0, atol=1e-12)
                np.testing.assert_allclose(a[1], b[1], rtol=0, atol=1e-12)


def test_planted_mask_bug_is_caught(monkeypatch):
    # A window mask that is one position too wide must break the mask/cache agreement.
    rng = np.random.default_rng(8)
    k, v = rand_hist(rng, 20, 1, 8)
    h = attn.array_history(k, v)
    q = rng.standard_normal((1, 8))
    good = attn.decode_query(q, 15, h, 2, 4, 1, 10000.0, 0.3)[0]

    def wide(P, W, p):
        j = np.arange(p + 1)
        return (j < P) | (j >= p - W)

    monkeypatch.setattr(attn, "visible_mask", wide)
    bad = attn.decode_query(q, 15, h, 2, 4, 1, 10000.0, 0.3)[0]
    ref = attn.decode_query_from_cache(q, 15, h, 2, 4, 1, 10000.0, 0.3)[0]
    np.testing.assert_allclose(good, ref, atol=1e-12)
    assert np.abs(bad - ref).max() > 1e-6


def test_zero_query_gives_mean_of_visible_values():
    rng = np.random.default_rng(9)
    P, W, p = 3, 5, 20
    k, v = rand_hist(rng, p + 1, 1, 8)
    out, lse = attn.decode_query(np.zeros((1, 8)), p, attn.array_history(k, v), P, W, 1, 10000.0, 0.5)
    vis = [j for j in range(p + 1) if spec.visible(P, W, p, j)]
    np.testing.assert_allclose(out[0], v[vis, 0].mean(axis=0), rtol=0, atol=1e-14)
    assert abs(lse[0] - np.log(len(vis))) < 1e-14


def test_first_token_returns_its_value():
    rng = np.random.default_rng(10)
    k, v = rand_hist(rng, 1, 2, 8)
    out, lse = attn.decode_query(rng.standard_normal((4, 8)), 0, attn.array_history(k, v), 4, 4, 2,
                                 10000.0, 0.5)
    np.testing.assert_array_equal(out, v[0][[0, 0, 1, 1]])


def test_constant_values_pass_through():
    rng = np.random.default_rng(11)
    n = 50
    k = rng.standard_normal((n, 1, 8))
    v = np.broadcast_to(rng.standard_normal(8), (n, 1, 8)).copy()
    out, _ = attn.decode_query(rng.standard_normal((2, 8)), n - 1, attn.array_history(k, v), 5, 7, 1,
                               10000.0, 0.5)
    np.testing.assert_allclose(out, np.broadcast_to(v[0, 0], (2, 8)), rtol=0, atol=1e-14)


def test_prefix_free_case_is_plain_sliding_window():
    # P = 0 is the plain sliding window of the Lean article: attention over lastWindow W of the
    # history, computed here from the list model with a softmax written out by hand.
    rng = np.random.default_rng(12)
    W, D = 6, 8
    n = 25
    k, v = rand_hist(rng, n, 1, D)
    for p in range(n):
        q = rng.standard_normal((1, D))
        win = spec.run(W, list(range(p + 1)))
        qr = rope.rotate(q, np.array([p]), 10000.0)[0]
        kr = rope.rotate(k[win, 0], np.array(win), 10000.0)
        s = kr @ qr * 0.4
        e = np.exp(s - s.max())
        ref = (e[:, None] * v[win, 0]).sum(0) / e.sum()
        out, _ = attn.decode_query(q, p, attn.array_history(k, v), 0, W, 1, 10000.0, 0.4)
        np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-13)


def test_masked_positions_cannot_leak():
    # Huge values at positions outside A(t) must not change the output at all.
    rng = np.random.default_rng(13)
    P, W, p = 4, 6, 40
    k, v = rand_hist(rng, p + 1, 2, 8)
    q = rng.standard_normal((2, 8))
    base = attn.decode_query(q, p, attn.array_history(k, v), P, W, 2, 10000.0, 0.3)[0]
    k2, v2 = k.copy(), v.copy()
    for j in range(p + 1):
        if not spec.visible(P, W, p, j):
            k2[j] = 1e6
            v2[j] = 1e6
    out = attn.decode_query(q, p, attn.array_history(k2, v2), P, W, 2, 10000.0, 0.3)[0]
    np.testing.assert_array_equal(out, base)


def test_grouped_heads_share_kv():
    rng = np.random.default_rng(14)
    k, v = rand_hist(rng, 30, 1, 8)
    q1 = rng.standard_normal((1, 8))
    q4 = np.repeat(q1, 4, axis=0)
    o1 = attn.decode_query(q1, 29, attn.array_history(k, v), 3, 10, 1, 10000.0, 0.3)[0]
    o4 = attn.decode_query(q4, 29, attn.array_history(k, v), 3, 10, 1, 10000.0, 0.3)[0]
    for h in range(4):
        np.testing.assert_array_equal(o4[h], o1[0])


def test_prefill_chunk_equals_single_steps():
    rng = np.random.default_rng(15)
    P, W, n, C = 3, 8, 20, 6
    k, v = rand_hist(rng, n + C, 2, 8)
    q = rng.standard_normal((C, 4, 8))
    h = attn.array_history(k, v)
    out, lse = attn.prefill_chunk(q, n, h, P, W, 2, 10000.0, 0.3)
    for c in range(C):
        o, s = attn.decode_query_from_cache(q[c], n + c, h, P, W, 2, 10000.0, 0.3)
        np.testing.assert_allclose(out[c], o, atol=1e-12)
        np.testing.assert_allclose(lse[c], s, atol=1e-12)
