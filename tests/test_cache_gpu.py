"""GPU cache contents against the list model, bit for bit.

After every append the exported logical view (prefix, then window oldest first) must
equal pinned_view(P, W, history): positions exact, V bytes exact, K bytes equal to
RNE(float64 rotation at the absolute position). Unfilled slots keep tag -1
([KV-Lean] 5.1). Walks every step up to 3W + P + 2, so the not-full, exactly-full and
first-replacement phases ([KV-Lean] 1.3) are all covered."""
import numpy as np
import pytest
import torch

from oracle import cache as ocache
from synth import configs, drive

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def dname(dtype):
    return "bf16" if dtype == torch.bfloat16 else "f32"


def check_seq(c, wl, b, n):
    k_e, v_e, pos_e = c.export(b)
    pos, kbits, v = ocache.expected_view(wl.prefix[b], wl.window, n, drive.hist_provider(wl, b),
                                         wl.rope_base, dname(wl.dtype))
    assert pos_e.tolist() == pos.tolist(), (b, n)
    np.testing.assert_array_equal(bits(k_e), kbits, err_msg=f"K bytes seq {b} n {n}")
    np.testing.assert_array_equal(v_e.double().numpy(), v, err_msg=f"V bytes seq {b} n {n}")
    tags = c.raw_tags()[b].cpu().numpy()
    assert (tags >= 0).sum() == len(pos)
    assert sorted(tags[tags >= 0].tolist()) == sorted(pos.tolist())


def small(P, W, dtype, B=2, D=64):
    prefix = [P, max(0, P - 2)][:B] + [P] * max(0, B - 2)
    wl = configs.Workload(f"small-P{P}-W{W}", dtype, B, 4, 2, D, W, prefix, [1] * B, "decode")
    return wl


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("P,W", [(0, 1), (0, 4), (3, 1), (3, 4), (2, 5), (4, 7)])
def test_every_step_single_token(P, W, dtype):
    wl = small(P, W, dtype)
    c = drive.make_cache(wl)
    for b in range(wl.batch):
        c.reset(b, wl.prefix[b])
    for n in range(1, 3 * W + P + 3):
        k, v = drive.kv_block(wl, [n - 1] * wl.batch, 1, "cuda")
        c.append(k, v)
        for b in range(wl.batch):
            check_seq(c, wl, b, n)
            assert c.seq_length(b) == n


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_multi_token_and_ragged_appends(dtype):
    # chunks longer than W evict inside one call; ragged counts leave some sequences idle
    W, D = 5, 128
    wl = configs.Workload("ragged", dtype, 3, 8, 4, D, W, [3, 0, 6], [1, 1, 1], "decode")
    c = drive.make_cache(wl)
    for b in range(3):
        c.reset(b, wl.prefix[b])
    n = [0, 0, 0]
    plan = [[1, 0, 2], [3, 7, 0], [W + 3, 1, 2 * W + 1], [0, 0, 0], [2, 12, 1], [W, W, W]]
    for counts in plan:
        stride = max(max(counts), 1)
        k = torch.empty((3, stride, 4, D), dtype=dtype, device="cuda")
        v = torch.empty_like(k)
        for b in range(3):
            kb, vb = drive.kv_block(wl, [n[b]] * 3, stride, "cuda")
            k[b], v[b] = kb[b], vb[b]
        c.append(k, v, n_new=counts)
        n = [a + b for a, b in zip(n, counts)]
        for b in range(3):
            check_seq(c, wl, b, n[b])


def test_resident_keys_never_change():
    # Continue PE ([PS] 05): a key is rotated once at its absolute position and then reused
    # unchanged for as long as it stays cached.
    wl = small(3, 6, torch.bfloat16, B=1, D=128)
    c = drive.make_cache(wl)
    c.reset(0, 3)
    seen = {}
    for n in range(1, 40):
        k, v = drive.kv_block(wl, [n - 1], 1, "cuda")
        c.append(k, v)
        k_e, _, pos_e = c.export(0)
        kb = bits(k_e)
        for i, p in enumerate(pos_e.tolist()):
            if p in seen:
                np.testing.assert_array_equal(seen[p], kb[i])
            else:
                seen[p] = kb[i].copy()


def test_reset_empties_a_sequence():
    wl = small(2, 4, torch.bfloat16)
    c = drive.make_cache(wl)
    for b in range(2):
        c.reset(b, wl.prefix[b])
    k, v = drive.kv_block(wl, [0, 0], 9, "cuda")
    c.append(k, v)
    c.reset(0, 1)
    assert c.seq_length(0) == 0
    assert (c.raw_tags()[0] == -1).all()
    _, _, pos = c.export(0)
    assert pos.numel() == 0
    wl2 = configs.Workload("re", torch.bfloat16, 2, 4, 2, 64, 4, [1, wl.prefix[1]], [1, 1], "decode")
    k, v = drive.kv_block(wl2, [0, 9], 6, "cuda")
    c.append(k, v, n_new=[6, 0])
    check_seq(c, wl2, 0, 6)
    check_seq(c, wl, 1, 9)


def test_tiny_fp32_cache_every_step():
    # The 200-step fp32 workload (P = 16, W = 32): the cache after every step.
    wl = configs.tiny_fp32()
    c = drive.make_cache(wl)
    c.reset(0, wl.prefix[0])
    for n in range(1, wl.steps + 1):
        k, v = drive.kv_block(wl, [n - 1], 1, "cuda")
        c.append(k, v)
        check_seq(c, wl, 0, n)


@pytest.mark.parametrize("D,base", [(64, 10000.0), (128, 10000.0), (128, 500000.0)])
def test_rotation_frequencies_are_the_nearest_doubles(D, base):
    # The cache's theta table (the library's work region starts with it) against the
    # oracle's correctly rounded base^(-2i/D), bit for bit: an angle p * theta_i of a late
    # position moves by p ulps of theta when theta is one ulp off.
    from oracle import rope
    wl = configs.Workload("theta", torch.bfloat16, 1, 8, 8, D, 16, [0], [1], "decode",
                          rope_base=base)
    c = drive.make_cache(wl)
    off = c.layout.work_offset
    got = c.mem[off:off + D // 2 * 8].cpu().numpy().view(np.float64)
    np.testing.assert_array_equal(got.view(np.uint64), rope.inv_freq(D, base).view(np.uint64))
