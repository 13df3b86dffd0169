"""Training attention forward and backward on the GPU against the float64 oracle.

Inputs are bf16 draws (exact in float64); the oracle recomputes everything in float64 from
them. The kernels round P and dS to bf16 before the second products and their outputs to
bf16; errors are measured relative to the largest reference magnitude of each output
(gradients have no fixed scale: a key's gradient sums over every query that sees it)."""
import numpy as np
import pytest
import torch

import prefix_pinned_sliding_amd as psa
from oracle import train
from synth import gen

pytestmark = pytest.mark.gpu

# bf16 tolerances: out as in the other attention tests; gradients relative to their scale.
# lse: the row sum is accumulated from the bf16-rounded probabilities that also weight V
# (so out stays a convex combination), which moves l by at most 2^-8 relative and lse by
# at most ln(1 + 2^-8) = 3.9e-3.
OUT_ABS, OUT_REL = 2e-2, 5e-3
GRAD_MAXREL, GRAD_REL = 2e-2, 1e-2
LSE_ABS = 5e-3


def draw(stream, B, T, H, D, seed=0):
    return gen.normal_block(seed, stream, list(range(B)), [0] * B, T, H, D, torch.bfloat16, "cuda")


def inputs(B, T, Hq, Hkv, D, seed=0):
    return (draw(gen.STREAM_Q, B, T, Hq, D, seed), draw(gen.STREAM_K, B, T, Hkv, D, seed),
            draw(gen.STREAM_V, B, T, Hkv, D, seed), draw(gen.STREAM_DO, B, T, Hq, D, seed))


def check_out(got, ref, what):
    err = np.abs(got - ref).max()
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= OUT_ABS and rel <= OUT_REL, f"{what}: max-abs {err} rel-l2 {rel}"


def check_grad(got, ref, what):
    scale = np.abs(ref).max()
    if scale == 0.0:
        # every row sees one key only (or nothing sees the key): the exact gradient is 0 and
        # the kernel's is dP - Di = <dO, v> - <dO, o> with o = v, a float32 rounding residue
        assert np.abs(got).max() <= 1e-4, f"{what}: expected 0, max-abs {np.abs(got).max()}"
        return
    err = np.abs(got - ref).max() / scale
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert err <= GRAD_MAXREL and rel <= GRAD_REL, f"{what}: max-abs/scale {err} rel-l2 {rel}"


CASES = [
    # B, T, Hq, Hkv, D, W, prefix, lens
    (3, 200, 4, 2, 128, 48, [10, 0, 70], [200, 163, 64]),
    (2, 131, 8, 8, 64, 33, [64, 5], [131, 1]),
    (2, 150, 8, 2, 64, 1, [3, 0], [150, 149]),
    (1, 300, 16, 2, 128, 300, [0], [300]),
    (2, 97, 8, 1, 128, 20, [97, 40], [97, 96]),
    # many key tiles and query steps: 17 key tiles, window and prefix both longer than a
    # tile, ragged lengths, G = 4 (D = 64) and G = 8 (D = 128)
    (2, 1100, 16, 4, 64, 300, [100, 37], [1100, 777]),
    (1, 900, 16, 2, 128, 200, [150], [900]),
]


@pytest.mark.parametrize("case", CASES, ids=[f"T{c[1]}-G{c[2] // c[3]}-D{c[4]}-W{c[5]}" for c in CASES])
def test_forward_and_backward(case):
    B, T, Hq, Hkv, D, W, prefix, lens = case
    q, k, v, g = inputs(B, T, Hq, Hkv, D)
    ta = psa.TrainAttention(B, T, Hq, Hkv, D, W)
    # rows >= len must stay untouched: fill outputs with a marker first
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, T, Hq), 7.0, dtype=torch.float32, device="cuda")
    ta.forward(q, k, v, prefix, lens, out=out, lse=lse)
    dq, dk, dv = (torch.full_like(x, 7.0) for x in (q, k, v))
    ta.backward(q, k, v, out, lse, g, prefix, lens, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    scale = 1.0 / np.sqrt(D)
    for b in range(B):
        n = lens[b]
        qa, ka, va, ga = (x[b, :n].double().cpu().numpy() for x in (q, k, v, g))
        ro, rl = train.forward(qa, ka, va, prefix[b], W, scale)
        check_out(out[b, :n].double().cpu().numpy(), ro, f"out seq {b}")
        np.testing.assert_allclose(lse[b, :n].cpu().numpy(), rl, rtol=0, atol=LSE_ABS)
        rq, rk, rv = train.backward(qa, ka, va, ga, prefix[b], W, scale)
        check_grad(dq[b, :n].double().cpu().numpy(), rq, f"dq seq {b}")
        check_grad(dk[b, :n].double().cpu().numpy(), rk, f"dk seq {b}")
        check_grad(dv[b, :n].double().cpu().numpy(), rv, f"dv seq {b}")
        for t in (out, dq, dk, dv):
            assert bool((t[b, n:] == 7.0).all()), f"rows beyond len written, seq {b}"
        assert bool((lse[b, n:] == 7.0).all())


def test_errors():
    ta = psa.TrainAttention(1, 8, 2, 1, 64, 4)
    q, k, v, g = inputs(1, 8, 2, 1, 64)
    with pytest.raises(psa.PsaError) as e:
        ta.forward(q, k, v, [0], [9])
    assert e.value.status == psa.PSA_ERR_ARG
    with pytest.raises(psa.PsaError) as e:
        ta.forward(q, k, v, [-1], None)
    assert e.value.status == psa.PSA_ERR_ARG
    with pytest.raises(psa.PsaError):
        psa.TrainAttention(1, 8, 3, 2, 64, 4)
    with pytest.raises(psa.PsaError):
        psa.TrainAttention(1, 8, 2, 1, 96, 4)


def test_truncated_segment_full_size_sampled():
    # The pages' truncated back-propagation shape: a 100-token prompt plus 4W = 16384 lead
    # tokens with W = 4096, 16/8 heads, D = 128. Sampled rows of one KV group against the
    # row-restricted oracle (prefix and window rows, the prefix edge and the last row).
    B, T, Hq, Hkv, D, W, P = 2, 100 + 4 * 4096, 16, 8, 128, 4096, 100
    q, k, v, g = inputs(B, T, Hq, Hkv, D, seed=3)
    ta = psa.TrainAttention(B, T, Hq, Hkv, D, W)
    out, lse = ta.forward(q, k, v, [P, P])
    dq, dk, dv = ta.backward(q, k, v, out, lse, g, [P, P])
    torch.cuda.synchronize()
    b, h = 1, 5
    G = Hq // Hkv
    hs = slice(h * G, (h + 1) * G)
    qa = q[b, :, hs].double().cpu().numpy()
    ga = g[b, :, hs].double().cpu().numpy()
    ka = k[b, :, h:h + 1].double().cpu().numpy()
    va = v[b, :, h:h + 1].double().cpu().numpy()
    scale = 1.0 / np.sqrt(D)
    rows = [0, 57, P - 1, P, P + 1, 4200, 9999, T - 1]
    ro, rl = train.forward_rows(qa, ka, va, P, W, scale, rows)
    check_out(out[b, rows, hs].double().cpu().numpy(), ro, "out rows")
    np.testing.assert_allclose(lse[b, rows, hs].cpu().numpy(), rl, rtol=0, atol=LSE_ABS)
    keys = [7, 5000, T - 1]
    rq, rk, rv = train.backward_rows(qa, ka, va, ga, P, W, scale, rows, keys)
    check_grad(dq[b, rows, hs].double().cpu().numpy(), rq, "dq rows")
    check_grad(dk[b, keys, h:h + 1].double().cpu().numpy(), rk, "dk rows")
    check_grad(dv[b, keys, h:h + 1].double().cpu().numpy(), rv, "dv rows")
