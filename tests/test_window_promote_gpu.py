"""Per-sequence window lengths and promotion into the pinned prefix, on the GPU.

The reference is the list model spec.WindowModel (w as a per-step parameter, promotion
moves the oldest window entries into the pinned list) and attention over its cache list
(attn.attend_view). Where the window length is constant per sequence, the closed-form
mask oracle with W = w_b is used instead. Cache contents are compared bit for bit after
every operation; attention outputs to the float tolerances of the other GPU tests."""
import copy

import numpy as np
import pytest
import torch

import prefix_pinned_sliding_amd as psa
from oracle import attn, spec
from oracle import cache as ocache
from synth import configs, drive

pytestmark = pytest.mark.gpu


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.int32).numpy().view(np.uint32)


def tol_check(out, ref, dtype, what=""):
    err = np.abs(out - ref).max()
    if dtype == torch.float32:
        assert err <= 1e-5, f"{what} max-abs {err}"
    else:
        rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
        assert err <= 2e-2 and rel <= 5e-3, f"{what} max-abs {err} rel-l2 {rel}"


def check_cache(c, wl, b, m, Pmax):
    """Export and raw tags of sequence b against the list model m."""
    view = np.asarray(m.view(), dtype=np.int64)
    k_e, v_e, pos_e = c.export(b)
    assert pos_e.tolist() == view.tolist(), (b, pos_e.tolist(), view.tolist())
    k, v = drive.hist_provider(wl, b)(view)
    dn = "bf16" if wl.dtype == torch.bfloat16 else "f32"
    np.testing.assert_array_equal(bits(k_e), ocache.stored_key_bits(k, view, wl.rope_base, dn),
                                  err_msg=f"K bytes seq {b}")
    np.testing.assert_array_equal(v_e.double().numpy(), v, err_msg=f"V bytes seq {b}")
    tags = c.raw_tags()[b].cpu().numpy()
    pre_tags = tags[:Pmax]
    assert pre_tags[pre_tags >= 0].tolist() == list(m.pinned), b
    assert (pre_tags[len(m.pinned):] == -1).all(), b
    ring = tags[Pmax:]
    assert sorted(ring[ring >= 0].tolist()) == list(m.window), (b, ring.tolist(), m.window)
    w, pinned, entries = c.window_info(b)
    assert (w, pinned, entries) == (m.w, len(m.pinned), len(m.window))


def append_rows(c, wl, n, counts):
    stride = max(max(counts), 1)
    k, v = drive.kv_block(wl, n, stride, "cuda")
    c.append(k, v, n_new=counts)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_random_operations_against_list_model(dtype, seed):
    # Appends (ragged, some longer than the window), window changes (shrink and growth) and
    # promotions in random order; cache bytes and tags after every operation, decode
    # against the list model's cache after every append.
    rng = np.random.default_rng(seed)
    W, Pmax, B = 12, 10, 3
    prefix = [3, 0, 5]
    wl = configs.Workload("wm", dtype, B, 8, 4, 64, W, prefix, [1] * B, "decode", seed=seed)
    c = drive.make_cache(wl, prefix_max=Pmax)
    models = []
    for b in range(B):
        c.reset(b, prefix[b])
        models.append(spec.WindowModel(prefix[b], W))
    n = [0] * B
    for step in range(60):
        op = rng.random()
        if op < 0.55 or step < 3:
            counts = [int(x) for x in rng.integers(0, 2 * W + 2, size=B)]
            if rng.random() < 0.5:
                counts = [int(x) for x in rng.integers(0, 3, size=B)]
            append_rows(c, wl, n, counts)
            for b in range(B):
                for p in range(n[b], n[b] + counts[b]):
                    models[b].push(p)
                n[b] += counts[b]
            if min(n) > 0:
                q = drive.queries(wl, [x - 1 for x in n], "cuda")
                out = c.decode(q).double().cpu().numpy()
                qc = q.double().cpu().numpy()
                for b in range(B):
                    ref, _ = attn.attend_view(qc[b], n[b] - 1, drive.hist_provider(wl, b),
                                              models[b].view(), wl.n_kv_heads, wl.rope_base,
                                              wl.scale)
                    tol_check(out[b], ref, dtype, f"step {step} seq {b}")
        elif op < 0.8:
            b = int(rng.integers(0, B))
            w = int(rng.integers(1, W + 1))
            c.set_window(b, w)
            models[b].set_window(w)
        else:
            b = int(rng.integers(0, B))
            room = Pmax - len(models[b].pinned)
            k = int(rng.integers(0, min(room, len(models[b].window)) + 1))
            c.promote(b, k)
            models[b].promote(k)
        for b in range(B):
            check_cache(c, wl, b, models[b], Pmax)


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 16, 8), (torch.bfloat16, 128, 32, 8),
                                            (torch.float32, 64, 8, 4), (torch.bfloat16, 64, 8, 8)])
@pytest.mark.parametrize("split", [0, 128])
def test_decode_ragged_windows(dtype, D, Hq, Hkv, split):
    # Constant per-sequence windows set at the start: the closed-form mask with W = w_b.
    W = 300
    prefix = [20, 0, 7, 100, 0, 64]
    wins = [1, 37, 128, 300, 200, 150]
    n_hist = [900, 36, 140, 1000, 250, 64 + 150 + 5]
    B = len(prefix)
    wl = configs.Workload("rw", dtype, B, Hq, Hkv, D, W, prefix, [1] * B, "decode")
    c = drive.make_cache(wl)
    c.set_split_tokens(split)
    for b in range(B):
        c.reset(b, prefix[b])
        c.set_window(b, wins[b])
    drive.fill(c, wl, n_hist, reset=False)
    k, v = drive.kv_block(wl, n_hist, 1, "cuda")
    c.append(k, v)
    q = drive.queries(wl, n_hist, "cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    out = c.decode(q, lse=lse).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(B):
        ref, rl = attn.decode_query(qc[b], n_hist[b], drive.hist_provider(wl, b), prefix[b],
                                    wins[b], Hkv, wl.rope_base, wl.scale)
        tol_check(out[b], ref, dtype, f"seq {b}")
        np.testing.assert_allclose(lse[b].cpu().numpy(), rl, rtol=0,
                                   atol=1e-5 if dtype == torch.float32 else 2e-2)


@pytest.mark.parametrize("split", [0, 128])
def test_decode_after_shrink_promote_and_growth(split):
    # Long histories: a shrink drops entries at once, promotion pins old window entries,
    # a growth refills only with new tokens; ring heads away from slot 0 and wrapping.
    W, Pmax = 700, 400
    prefix = [50, 0, 300, 10]
    wl = configs.Workload("spg", torch.bfloat16, 4, 16, 8, 128, W, prefix, [1] * 4, "decode")
    c = drive.make_cache(wl, prefix_max=Pmax)
    c.set_split_tokens(split)
    models = [spec.WindowModel(p, W) for p in prefix]
    n = [1500, 900, 2000, 650]
    drive.fill(c, wl, n)
    for b in range(4):
        for p in range(n[b]):
            models[b].push(p)
    ops = [(0, "w", 333), (1, "p", 90), (2, "w", 129), (2, "p", 100), (3, "p", 390),
           (3, "w", 5)]
    for b, kind, x in ops:
        if kind == "w":
            c.set_window(b, x)
            models[b].set_window(x)
        else:
            c.promote(b, x)
            models[b].promote(x)
    for b in range(4):
        check_cache(c, wl, b, models[b], Pmax)
    for b, w in ((0, 700), (3, 400)):
        c.set_window(b, w)
        models[b].set_window(w)
    for rounds in range(3):
        add = [257, 1, 64, 390]
        append_rows(c, wl, n, add)
        for b in range(4):
            for p in range(n[b], n[b] + add[b]):
                models[b].push(p)
            n[b] += add[b]
            check_cache(c, wl, b, models[b], Pmax)
        q = drive.queries(wl, [x - 1 for x in n], "cuda")
        out = c.decode(q).double().cpu().numpy()
        qc = q.double().cpu().numpy()
        for b in range(4):
            ref, _ = attn.attend_view(qc[b], n[b] - 1, drive.hist_provider(wl, b),
                                      models[b].view(), wl.n_kv_heads, wl.rope_base, wl.scale)
            tol_check(out[b], ref, torch.bfloat16, f"round {rounds} seq {b}")


def prefill_reference(wl, b, m, n, qc, pe="continue"):
    m = copy.deepcopy(m)
    hist = drive.hist_provider(wl, b)
    outs = []
    for r in range(qc.shape[0]):
        m.push(n + r)
        o, _ = attn.attend_view(qc[r], n + r, hist, m.view(), wl.n_kv_heads, wl.rope_base,
                                wl.scale, pe)
        outs.append(o)
    return np.stack(outs)


@pytest.mark.parametrize("C", [128, 77])
def test_prefill_with_window_changes(C):
    W, Pmax = 96, 120
    prefix = [40, 10, 0, 30, 100]
    n = [20, 300, 250, 260, 180]
    B = len(prefix)
    wl = configs.Workload("pfw", torch.bfloat16, B, 16, 8, 128, W, prefix, [1] * B, "prefill")
    c = drive.make_cache(wl, max_chunk=C, prefix_max=Pmax)
    models = [spec.WindowModel(p, W) for p in prefix]
    for b in range(B):
        c.reset(b, prefix[b])
    c.set_window(0, 40)            # prefix still filling: the chunk crosses P_0
    models[0].set_window(40)
    drive.fill(c, wl, n, reset=False)
    for b in range(B):
        for p in range(n[b]):
            models[b].push(p)
    for b, kind, x in [(1, "w", 30), (2, "p", 64), (2, "w", 17), (3, "w", 8), (3, "w", 90),
                       (4, "p", 20)]:
        if kind == "w":
            c.set_window(b, x)
            models[b].set_window(x)
        else:
            c.promote(b, x)
            models[b].promote(x)
    q = drive.query_block(wl, n, C, "cuda")
    k, v = drive.kv_block(wl, n, C, "cuda")
    out = c.prefill(q, k, v).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(B):
        ref = prefill_reference(wl, b, models[b], n[b], qc[b])
        tol_check(out[b], ref, torch.bfloat16, f"prefill seq {b}")
        for p in range(n[b], n[b] + C):
            models[b].push(p)
        check_cache(c, wl, b, models[b], Pmax)


def test_reset_pe_with_window_changes():
    # RESET numbers the attended list [prefix, window] 0 .. len - 1; with a changed window
    # length the window part is whatever the list model holds.
    W, C = 80, 64
    prefix = [30, 0, 12]
    n = [200, 150, 20]
    B = 3
    wl = configs.Workload("rpw", torch.bfloat16, B, 16, 8, 128, W, prefix, [1] * B, "prefill")
    c = drive.make_cache(wl, max_chunk=C, pe="reset")
    models = [spec.WindowModel(p, W) for p in prefix]
    for b in range(B):
        c.reset(b, prefix[b])
    c.set_window(2, 25)
    models[2].set_window(25)
    drive.fill(c, wl, n, reset=False)
    for b in range(B):
        for p in range(n[b]):
            models[b].push(p)
    c.set_window(0, 33)
    models[0].set_window(33)
    c.set_window(1, 9)
    models[1].set_window(9)
    c.set_window(1, 50)
    models[1].set_window(50)
    q = drive.query_block(wl, n, C, "cuda")
    k, v = drive.kv_block(wl, n, C, "cuda")
    out = c.prefill(q, k, v).double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for b in range(B):
        ref = prefill_reference(wl, b, models[b], n[b], qc[b], pe="reset")
        tol_check(out[b], ref, torch.bfloat16, f"reset prefill seq {b}")
        for p in range(n[b], n[b] + C):
            models[b].push(p)
    kd, vd = drive.kv_block(wl, [x + C for x in n], 1, "cuda")
    c.append(kd, vd)
    qd = drive.queries(wl, [x + C for x in n], "cuda")
    outd = c.decode(qd).double().cpu().numpy()
    qdc = qd.double().cpu().numpy()
    for b in range(B):
        models[b].push(n[b] + C)
        ref, _ = attn.attend_view(qdc[b], n[b] + C, drive.hist_provider(wl, b), models[b].view(),
                                  wl.n_kv_heads, wl.rope_base, wl.scale, "reset")
        tol_check(outd[b], ref, torch.bfloat16, f"reset decode seq {b}")


def test_errors_leave_the_cache_unchanged():
    W, Pmax = 16, 8
    wl = configs.Workload("err", torch.bfloat16, 2, 8, 4, 64, W, [4, 4], [1, 1], "decode")
    c = drive.make_cache(wl, prefix_max=Pmax, n_shared=1, shared_max=8)
    with pytest.raises(psa.PsaError) as e:
        c.set_window(0, 5)
    assert e.value.status == psa.PSA_ERR_STATE          # never reset
    c.reset(0, 4)
    kp, vp = drive.kv_rows_from(wl, [1], [0], 4, "cuda")
    c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())
    c.attach(1, 0)
    m = spec.WindowModel(4, W)
    k, v = drive.kv_block(wl, [0, 4], 30, "cuda")
    c.append(k, v, n_new=[30, 0])
    for p in range(30):
        m.push(p)
    before = c.export(0)
    for bad in (0, W + 1, -3):
        with pytest.raises(psa.PsaError) as e:
            c.set_window(0, bad)
        assert e.value.status == psa.PSA_ERR_ARG
    for bad in (-1, Pmax - 4 + 1, W + 1):
        with pytest.raises(psa.PsaError) as e:
            c.promote(0, bad)
        assert e.value.status == psa.PSA_ERR_ARG
    with pytest.raises(psa.PsaError) as e:
        c.promote(1, 1)
    assert e.value.status == psa.PSA_ERR_STATE          # reads a shared prefix
    after = c.export(0)
    for x, y in zip(before, after):
        assert torch.equal(x, y)
    check_cache(c, wl, 0, m, Pmax)
    c.set_window(1, 3)                                   # allowed on an attached sequence
    assert c.window_info(1) == (3, 4, 0)
    # a reset restores the full window
    c.set_window(0, 2)
    c.reset(0, 4)
    assert c.window_info(0) == (W, 0, 0)
    rc = drive.make_cache(wl, prefix_max=Pmax, pe="reset")
    rc.reset(0, 0)
    kr, vr = drive.kv_block(wl, [0, 0], 3, "cuda")
    rc.append(kr, vr, n_new=[3, 0])
    with pytest.raises(psa.PsaError) as e:
        rc.promote(0, 1)
    assert e.value.status == psa.PSA_ERR_STATE          # RESET numbering has no promotion
