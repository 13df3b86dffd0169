"""Pins of oracle/train.py: masked attention forward and backward in float64.

Independent of the formulas in the oracle: torch's float64 scaled-dot-product attention
with a boolean mask for the forward, torch.autograd through that forward for the
gradients, central finite differences of the loss, and two exact identities of the
softmax Jacobian (per query its rows sum to zero, so key gradients sum to zero; softmax
rows sum to one, so value gradients sum to the output gradients)."""
import numpy as np
import pytest
import torch

from oracle import spec, train


def rnd(rng, *shape):
    return rng.standard_normal(shape)


def test_row_mask_is_the_visible_set():
    # rows >= P are consecutive positions: the row mask equals A(t) in position space
    for P in range(0, 5):
        for W in range(1, 6):
            m = train.row_mask(14, P, W)
            for i in range(14):
                vis = set(np.nonzero(m[i])[0].tolist())
                assert vis == {t - 1 for t in spec.visible_1based(P, W, i + 1)}


def torch_forward(q, k, v, P, W, scale):
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    mask = torch.as_tensor(train.row_mask(T, P, W))
    qh = q.permute(1, 0, 2)
    kh = k.repeat_interleave(G, dim=1).permute(1, 0, 2)
    vh = v.repeat_interleave(G, dim=1).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2)


@pytest.mark.parametrize("T,P,W,Hq,Hkv", [(20, 3, 5, 4, 2), (17, 0, 4, 2, 2), (24, 24, 3, 4, 1),
                                          (30, 6, 40, 8, 2), (16, 2, 1, 2, 1)])
def test_forward_and_backward_against_autograd(T, P, W, Hq, Hkv):
    rng = np.random.default_rng(T * 7 + P)
    D, scale = 8, 0.37
    q, k, v, g = rnd(rng, T, Hq, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hq, D)
    out, lse = train.forward(q, k, v, P, W, scale)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch_forward(tq, tk, tv, P, W, scale)
    np.testing.assert_allclose(out, to.detach().numpy(), rtol=0, atol=1e-12)
    (to * torch.tensor(g)).sum().backward()
    dq, dk, dv = train.backward(q, k, v, g, P, W, scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-11)
    # lse: the log normaliser, checked against a direct log-sum-exp over visible keys
    G = Hq // Hkv
    mask = train.row_mask(T, P, W)
    for i in (0, T // 2, T - 1):
        for hq in range(Hq):
            z = scale * (k[mask[i], hq // G, :] @ q[i, hq, :])
            assert abs(lse[i, hq] - np.log(np.exp(z).sum())) < 1e-12


def test_backward_against_finite_differences():
    rng = np.random.default_rng(5)
    T, P, W, Hq, Hkv, D, scale = 11, 2, 4, 4, 2, 4, 0.8
    q, k, v, g = rnd(rng, T, Hq, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hq, D)
    dq, dk, dv = train.backward(q, k, v, g, P, W, scale)

    def loss(q_, k_, v_):
        return float(np.sum(train.forward(q_, k_, v_, P, W, scale)[0] * g))

    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0), (1, 1, 3), (5, 0, 2), (T - 1, 1, 1), (P, 0, 0), (T - 3, 1, 2)]:
            idx = idx[:1] + (idx[1] % x.shape[1],) + idx[2:]
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7, (name, idx, fd, grad[idx])


def test_gradient_identities():
    rng = np.random.default_rng(9)
    T, P, W, Hq, Hkv, D = 40, 5, 7, 8, 2, 16
    q, k, v, g = rnd(rng, T, Hq, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hq, D)
    dq, dk, dv = train.backward(q, k, v, g, P, W, 0.25)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-11)
    G = Hq // Hkv
    for hk in range(Hkv):
        np.testing.assert_allclose(dv[:, hk, :].sum(axis=0),
                                   g[:, hk * G:(hk + 1) * G, :].sum(axis=(0, 1)), atol=1e-11)
    # keys no query sees get no gradient: with P = 0 and W = 1 each row sees only itself
    dq1, dk1, dv1 = train.backward(q, k, v, g, 0, 1, 0.25)
    np.testing.assert_allclose(dq1, 0.0, atol=1e-12)      # softmax over one key is constant
    np.testing.assert_allclose(dk1, 0.0, atol=1e-12)
    np.testing.assert_allclose(dv1, g.reshape(T, Hkv, G, D).sum(axis=2), atol=1e-12)


def test_row_restricted_forms_equal_the_full_ones():
    rng = np.random.default_rng(13)
    T, P, W, Hq, Hkv, D = 37, 6, 9, 4, 2, 8
    q, k, v, g = rnd(rng, T, Hq, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hkv, D), rnd(rng, T, Hq, D)
    out, lse = train.forward(q, k, v, P, W, 0.3)
    dq, dk, dv = train.backward(q, k, v, g, P, W, 0.3)
    rows = [0, 3, 5, 6, 7, 20, 36]
    o2, l2 = train.forward_rows(q, k, v, P, W, 0.3, rows)
    np.testing.assert_allclose(o2, out[rows], rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse[rows], rtol=0, atol=1e-12)
    dq2, dk2, dv2 = train.backward_rows(q, k, v, g, P, W, 0.3, rows, rows)
    np.testing.assert_allclose(dq2, dq[rows], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk2, dk[rows], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv2, dv[rows], rtol=0, atol=1e-11)
