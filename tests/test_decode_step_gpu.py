"""The fused decode step (psa_decode_step) on the GPU.

[PS] 03's generation loop appends the new token, then attends to the prefix and the window.
psa_decode_step does both in one decode launch, so it must leave exactly what
psa_append(one token) followed by psa_decode_attn leaves. Each test drives two caches side
by side, one with the two calls and one with the fused call, and compares:
* outputs and lse exactly (the attention arithmetic is the same code in the same order);
* the exported caches (keys, values, positions) and the raw tags bit for bit;
* the outputs against the float64 oracle, to the bf16 / fp32 tolerances of the other tests.
The steps run from an empty sequence through the prefix fill, a window that is not full,
the first eviction and many more, in both layouts and both position modes."""
import numpy as np
import pytest
import torch

from oracle import attn, spec
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


def same_state(a, b, B):
    for s in range(B):
        ea, eb = a.export(s), b.export(s)
        assert ea[2].tolist() == eb[2].tolist(), f"positions seq {s}"
        np.testing.assert_array_equal(bits(ea[0]), bits(eb[0]), err_msg=f"K seq {s}")
        np.testing.assert_array_equal(bits(ea[1]), bits(eb[1]), err_msg=f"V seq {s}")
        assert a.seq_length(s) == b.seq_length(s)
    assert torch.equal(a.raw_tags(), b.raw_tags())


def twin_steps(wl, caches, n, steps, models=None, check_every=7, split=0):
    """Run `steps` decode steps on caches = (two-call cache, fused cache) from lengths n."""
    two, fused = caches
    B = wl.batch
    for c in caches:
        if split:
            c.set_split_tokens(split)
    for step in range(steps):
        k, v = drive.kv_block(wl, n, 1, "cuda")
        q = drive.queries(wl, n, "cuda")
        lt = torch.empty((B, wl.n_q_heads), dtype=torch.float32, device="cuda")
        lf = torch.empty_like(lt)
        two.append(k, v)
        ot = two.decode(q, lse=lt)
        of = fused.decode_step(k[:, 0].contiguous(), v[:, 0].contiguous(), q, lse=lf)
        assert torch.equal(ot, of), f"step {step}: outputs differ"
        assert torch.equal(lt, lf), f"step {step}: lse differ"
        n = [x + 1 for x in n]
        if models is not None:
            for s in range(B):
                models[s].push(n[s] - 1)
        if step % check_every == 0 or step == steps - 1:
            same_state(two, fused, B)
            out = of.double().cpu().numpy()
            qc = q.double().cpu().numpy()
            for s in range(B):
                if models is not None:
                    ref, _ = attn.attend_view(qc[s], n[s] - 1, drive.hist_provider(wl, s),
                                              models[s].view(), wl.n_kv_heads, wl.rope_base,
                                              wl.scale)
                else:
                    ref, _ = attn.decode_query(qc[s], n[s] - 1, drive.hist_provider(wl, s),
                                               wl.prefix[s], wl.window, wl.n_kv_heads,
                                               wl.rope_base, wl.scale, pe=fused.pe)
                tol_check(out[s], ref, wl.dtype, f"step {step} seq {s}")
    return n


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [(torch.bfloat16, 128, 16, 8), (torch.bfloat16, 64, 32, 8),
                                            (torch.float32, 64, 4, 4), (torch.bfloat16, 128, 8, 8)])
@pytest.mark.parametrize("block_size", [0, 16])
def test_from_empty_through_eviction(dtype, D, Hq, Hkv, block_size):
    W, Pmax = 48, 32
    prefix = [16, 0, 32]
    wl = configs.Workload("step", dtype, 3, Hq, Hkv, D, W, prefix, [1] * 3, "decode")
    caches = [drive.make_cache(wl, prefix_max=Pmax, block_size=block_size) for _ in range(2)]
    for c in caches:
        for s in range(3):
            c.reset(s, prefix[s])
    twin_steps(wl, caches, [0, 0, 0], 2 * W + Pmax + 5)


@pytest.mark.parametrize("pe", ["continue", "reset"])
@pytest.mark.parametrize("split", [0, 128])
def test_full_rings_over_several_splits(pe, split):
    # A full ring is read from slot 0, so the new token's slot (the evicted entry's) falls
    # in any split as the steps go on; sequence 0 also crosses the end of its prefix.
    W, Pmax = 200, 100
    prefix = [100, 37, 0]
    wl = configs.Workload("step-rp", torch.bfloat16, 3, 16, 8, 128, W, prefix, [1] * 3, "decode")
    caches = [drive.make_cache(wl, prefix_max=Pmax, pe=pe) for _ in range(2)]
    n0 = [90, 400, 260]
    for c in caches:
        drive.fill(c, wl, n0)
    twin_steps(wl, caches, n0, 220, split=split, check_every=23)


def test_window_changes_and_promotion():
    # per-sequence windows and promoted entries: the step's tag clearing and slots follow
    # the same rules as the append kernel
    W, Pmax = 64, 48
    prefix = [8, 0, 20]
    wl = configs.Workload("step-w", torch.bfloat16, 3, 8, 4, 64, W, prefix, [1] * 3, "decode")
    caches = [drive.make_cache(wl, prefix_max=Pmax) for _ in range(2)]
    models = [spec.WindowModel(p, W) for p in prefix]
    n0 = [150, 90, 30]
    for c in caches:
        drive.fill(c, wl, n0)
    for s in range(3):
        for p in range(n0[s]):
            models[s].push(p)
    for c in caches:
        c.set_window(0, 17)
        c.set_window(2, 40)
        c.promote(1, 5)
    models[0].set_window(17)
    models[2].set_window(40)
    models[1].promote(5)
    n = twin_steps(wl, caches, n0, 30, models=models)
    for c in caches:
        c.set_window(0, 64)
        c.set_window(1, 9)
    models[0].set_window(64)
    models[1].set_window(9)
    twin_steps(wl, caches, n, 30, models=models)


def test_shared_prefix():
    W, P = 64, 90
    wl = configs.Workload("step-sh", torch.bfloat16, 2, 16, 8, 128, W, [P, P], [1, 1], "decode")
    caches = [drive.make_cache(wl, n_shared=1, shared_max=P, prefix_max=0) for _ in range(2)]
    kp, vp = drive.kv_rows_from(wl, [0], [0], P, "cuda")
    k, v = drive.kv_rows_from(wl, [0, 1], [P, P], 70, "cuda")
    for c in caches:
        c.prefix_load(0, kp[0].contiguous(), vp[0].contiguous())
        c.attach(0, 0)
        c.attach(1, 0)
        c.append(k, v)
    two, fused = caches
    n = P + 70
    for step in range(20):
        kk, vv = drive.kv_rows_from(wl, [0, 1], [n, n], 1, "cuda")
        q = drive.queries(wl, [n, n], "cuda")
        two.append(kk, vv)
        ot = two.decode(q)
        of = fused.decode_step(kk[:, 0].contiguous(), vv[:, 0].contiguous(), q)
        assert torch.equal(ot, of), f"step {step}"
        n += 1
    same_state(two, fused, 2)
    qc = q.double().cpu().numpy()
    out = of.double().cpu().numpy()
    for s in range(2):
        hist = drive.composite_history(wl, 0, s, P)
        ref, _ = attn.decode_query(qc[s], n - 1, hist, P, W, wl.n_kv_heads, wl.rope_base, wl.scale)
        tol_check(out[s], ref, torch.bfloat16, f"seq {s}")


def test_errors_leave_the_state_unchanged():
    W = 32
    wl = configs.Workload("step-e", torch.bfloat16, 2, 8, 4, 64, W, [4, 4], [1, 1], "decode")
    c = drive.make_cache(wl, prefix_max=16)
    c.reset(0, 4)                             # sequence 1 never reset
    k, v = drive.kv_block(wl, [0, 0], 1, "cuda")
    q = drive.queries(wl, [0, 0], "cuda")
    with pytest.raises(RuntimeError):
        c.decode_step(k[:, 0].contiguous(), v[:, 0].contiguous(), q)
    assert c.seq_length(0) == 0
    with pytest.raises(ValueError):
        c.decode_step(k.contiguous(), v.contiguous(), q)      # [B][1][H][D] is not [B][H][D]


def test_default_workload_full_size():
    # the default decode workload (64 sequences at t = 32768, P = 100, W = 4096): several
    # fused steps, outputs equal to the two-call path bit for bit (their parity with the
    # oracle over the whole tensor is test_full_size_gpu.py's)
    wl = configs.decode_p100_w4096()
    n0 = [t - 1 for t in wl.start]
    caches = [drive.make_cache(wl) for _ in range(2)]
    for c in caches:
        drive.fill(c, wl, n0)
    two, fused = caches
    n = list(n0)
    for step in range(3):
        k, v = drive.kv_block(wl, n, 1, "cuda")
        q = drive.queries(wl, n, "cuda")
        two.append(k, v)
        ot = two.decode(q)
        of = fused.decode_step(k[:, 0].contiguous(), v[:, 0].contiguous(), q)
        assert torch.equal(ot, of), f"step {step}"
        n = [x + 1 for x in n]
    same_state(two, fused, wl.batch)
