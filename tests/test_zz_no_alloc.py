"""psa_train_bwd_noalloc (the backward pass with its scratch in the library's static device
array, for callers that cannot allocate) against psa_train_bwd (caller workspace) through
the C-ABI: bit-identical gradients on two calls in a row, the second with a smaller input
that leaves the first call's contents in the static array."""
import pytest
import torch

import prefix_pinned_sliding_amd as psa
from synth import gen

pytestmark = pytest.mark.gpu


def draw(B, T, H, D, stream, seed):
    return gen.normal_block(seed, stream, list(range(B)), [0] * B, T, H, D, torch.bfloat16, "cuda")


def case(B, T, Hq, Hkv, D, W, prefix, lens, seed):
    print(f"no-alloc backward: B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} W={W} prefix={prefix} "
          f"lens={lens}", flush=True)
    q, k, v = draw(B, T, Hq, D, gen.STREAM_Q, seed), draw(B, T, Hkv, D, gen.STREAM_K, seed), \
        draw(B, T, Hkv, D, gen.STREAM_V, seed)
    g = draw(B, T, Hq, D, gen.STREAM_DO, seed)
    ta = psa.TrainAttention(B, T, Hq, Hkv, D, W)
    out, lse = ta.forward(q, k, v, prefix, lens)
    grads = [torch.full_like(x, float("nan")) for x in (q, k, v)]
    ta.backward_noalloc(q, k, v, out, lse, g, prefix, lens, *grads)
    want = ta.backward(q, k, v, out, lse, g, prefix, lens)
    torch.cuda.synchronize()
    for name, a, b, n in zip(("dq", "dk", "dv"), grads, want, (Hq, Hkv, Hkv)):
        for bb in range(B):
            rows = T if lens is None else lens[bb]
            assert torch.equal(a[bb, :rows], b[bb, :rows]), f"{name} sequence {bb}"


def test_noalloc_backward_equals_workspace_backward():
    case(3, 700, 16, 8, 128, 256, [100, 0, 700], [700, 450, 700], seed=3)
    case(1, 129, 8, 2, 64, 40, [5], None, seed=4)
