"""Paged K/V storage on the GPU: a pool of blocks read through per-sequence block tables.

[KV-Lean] 6.1 frames a paged cache as the same logical cache read through a table of
physical blocks. So after every operation a paged cache must hold the same logical contents
and give the same attention as a contiguous one. Each test runs one sequence of operations
on a contiguous and a paged cache side by side:
* exports are compared bit for bit;
* decode and prefill outputs are compared exactly (the kernels do the same arithmetic in
  the same order; only row addresses differ);
* the list model and the float64 oracle are checked as in the other GPU tests.
The block allocator is checked through its invariants: every logical block that holds a
cached entry is mapped, no physical block is mapped twice, and mapped + free = n_blocks."""
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


def same_export(a, b, B):
    for s in range(B):
        ea, eb = a.export(s), b.export(s)
        assert ea[2].tolist() == eb[2].tolist(), f"positions seq {s}"
        np.testing.assert_array_equal(bits(ea[0]), bits(eb[0]), err_msg=f"K seq {s}")
        np.testing.assert_array_equal(bits(ea[1]), bits(eb[1]), err_msg=f"V seq {s}")
    assert torch.equal(a.raw_tags(), b.raw_tags())


def check_blocks(c, B):
    used = []
    free = None
    tags = c.raw_tags().cpu().numpy()
    Bs = c.block_size
    for s in range(B):
        table, free = c.blocks(s)
        assert len(table) == c.layout.slots // Bs
        for j, blk in enumerate(table):
            if (tags[s, j * Bs:(j + 1) * Bs] >= 0).any():
                assert blk >= 0, f"seq {s}: logical block {j} holds entries but is unmapped"
        used += [blk for blk in table if blk >= 0]
    assert len(used) == len(set(used)), "a physical block is mapped twice"
    assert all(0 <= blk < c.layout.n_blocks for blk in used)
    assert len(used) + free == c.layout.n_blocks


def check_model(c, wl, s, m):
    view = np.asarray(m.view(), dtype=np.int64)
    k_e, v_e, pos_e = c.export(s)
    assert pos_e.tolist() == view.tolist()
    k, v = drive.hist_provider(wl, s)(view)
    dn = "bf16" if wl.dtype == torch.bfloat16 else "f32"
    np.testing.assert_array_equal(bits(k_e), ocache.stored_key_bits(k, view, wl.rope_base, dn))
    np.testing.assert_array_equal(v_e.double().numpy(), v)


@pytest.mark.parametrize("dtype,Bs", [(torch.bfloat16, 16), (torch.float32, 16), (torch.bfloat16, 32)])
@pytest.mark.parametrize("seed", [0, 1])
def test_random_operations_paged_equals_contiguous(dtype, Bs, seed):
    # Ragged appends (some longer than the window), window changes, promotions and resets in
    # random order; after every operation the two caches agree and the allocator invariants
    # hold; decode is compared exactly and against the list model's cache.
    rng = np.random.default_rng(100 + seed)
    W, Pmax, B = 64, 32, 3
    prefix = [5, 0, 20]
    wl = configs.Workload("pg", dtype, B, 8, 4, 64, W, prefix, [1] * B, "decode", seed=seed)
    cc = drive.make_cache(wl, prefix_max=Pmax)
    pc = drive.make_cache(wl, prefix_max=Pmax, block_size=Bs)
    models = [spec.WindowModel(p, W) for p in prefix]
    for s in range(B):
        cc.reset(s, prefix[s])
        pc.reset(s, prefix[s])
    n = [0] * B
    for step in range(50):
        op = rng.random()
        if op < 0.55 or step < 3:
            counts = [int(x) for x in rng.integers(0, 2 * W + 2, size=B)]
            if rng.random() < 0.5:
                counts = [int(x) for x in rng.integers(0, 3, size=B)]
            k, v = drive.kv_block(wl, n, max(max(counts), 1), "cuda")
            cc.append(k, v, n_new=counts)
            pc.append(k, v, n_new=counts)
            for s in range(B):
                for p in range(n[s], n[s] + counts[s]):
                    models[s].push(p)
                n[s] += counts[s]
            if min(n) > 0:
                q = drive.queries(wl, [x - 1 for x in n], "cuda")
                lc = torch.empty((B, wl.n_q_heads), dtype=torch.float32, device="cuda")
                lp = torch.empty_like(lc)
                oc = cc.decode(q, lse=lc)
                op_ = pc.decode(q, lse=lp)
                assert torch.equal(oc, op_) and torch.equal(lc, lp), f"step {step}"
                out = op_.double().cpu().numpy()
                qc = q.double().cpu().numpy()
                for s in range(B):
                    ref, _ = attn.attend_view(qc[s], n[s] - 1, drive.hist_provider(wl, s),
                                              models[s].view(), wl.n_kv_heads, wl.rope_base,
                                              wl.scale)
                    tol_check(out[s], ref, dtype, f"step {step} seq {s}")
        elif op < 0.75:
            s = int(rng.integers(0, B))
            w = int(rng.integers(1, W + 1))
            cc.set_window(s, w)
            pc.set_window(s, w)
            models[s].set_window(w)
        elif op < 0.92:
            s = int(rng.integers(0, B))
            room = Pmax - len(models[s].pinned)
            kk = int(rng.integers(0, min(room, len(models[s].window)) + 1))
            cc.promote(s, kk)
            pc.promote(s, kk)
            models[s].promote(kk)
        else:                                   # a reset returns the sequence's blocks
            s = int(rng.integers(0, B))
            cc.reset(s, prefix[s])
            pc.reset(s, prefix[s])
            models[s] = spec.WindowModel(prefix[s], W)
            n[s] = 0
        same_export(cc, pc, B)
        check_blocks(pc, B)
        for s in range(B):
            check_model(pc, wl, s, models[s])


@pytest.mark.parametrize("pe", ["continue", "reset"])
@pytest.mark.parametrize("C", [64, 100])
def test_prefill_paged_equals_contiguous(pe, C):
    W, Pmax, Bs = 128, 64, 32
    prefix = [10, 0, 64, 30]
    n = [20, 300, 250, 700]
    B = len(prefix)
    wl = configs.Workload("pgp", torch.bfloat16, B, 16, 8, 128, W, prefix, [1] * B, "prefill")
    caches = [drive.make_cache(wl, max_chunk=C, prefix_max=Pmax, pe=pe),
              drive.make_cache(wl, max_chunk=C, prefix_max=Pmax, pe=pe, block_size=Bs)]
    for c in caches:
        for s in range(B):
            c.reset(s, prefix[s])
        c.set_window(0, 40)
        drive.fill(c, wl, n, reset=False)
        c.set_window(1, 100)
        if pe == "continue":
            c.promote(3, 20)
    pos = list(n)
    for rnd in range(3):
        q = drive.query_block(wl, pos, C, "cuda")
        k, v = drive.kv_block(wl, pos, C, "cuda")
        lse = [torch.empty((B, C, 16), dtype=torch.float32, device="cuda") for _ in caches]
        outs = [c.prefill(q, k, v, lse=l) for c, l in zip(caches, lse)]
        assert torch.equal(outs[0], outs[1]), f"round {rnd}"
        assert torch.equal(lse[0], lse[1]), f"round {rnd}"
        pos = [p + C for p in pos]
        same_export(caches[0], caches[1], B)
        check_blocks(caches[1], B)
    # the paged prefill against the oracle directly, on one sequence (plain window)
    s = 2
    qc = q.double().cpu().numpy()[s]
    out = outs[1].double().cpu().numpy()[s]
    hist = drive.hist_provider(wl, s)
    for r in (0, C // 2, C - 1):
        mm = spec.WindowModel(prefix[s], W)
        for p in range(pos[s] - C + r + 1):
            mm.push(p)
        ref, _ = attn.attend_view(qc[r], pos[s] - C + r, hist, mm.view(), wl.n_kv_heads,
                                  wl.rope_base, wl.scale, pe)
        tol_check(out[r], ref, torch.bfloat16, f"row {r}")


def test_shared_prefix_with_paged_window():
    # 8 runs of one 64-token prompt: the prompt lives once in the shared-prefix pool, the
    # windows in pool blocks; attached sequences hold no prefix blocks.
    W, Bs = 256, 64
    wl = configs.Workload("pgs", torch.bfloat16, 8, 16, 8, 128, W, [64] * 8, [1] * 8, "decode")
    n_hist = [64 + 17 * b + 1 for b in range(8)]
    n_hist[3] = 64 + 2 * W + 5
    caches = [drive.make_cache(wl, n_shared=1, shared_max=64, prefix_max=64),
              drive.make_cache(wl, n_shared=1, shared_max=64, prefix_max=64, block_size=Bs)]
    for c in caches:
        drive.fill_one_prompt(c, wl, n_hist, shared=True)
    for s in range(8):
        table, _ = caches[1].blocks(s)
        assert all(t == -1 for t in table[:64 // Bs]), "attached sequence holds prefix blocks"
    q = drive.queries(wl, [x - 1 for x in n_hist], "cuda")
    o0, o1 = caches[0].decode(q), caches[1].decode(q)
    assert torch.equal(o0, o1)
    same_export(caches[0], caches[1], 8)
    check_blocks(caches[1], 8)
    hist = drive.composite_history(wl, 0, 3, 64)
    ref, _ = attn.decode_query(q[3].double().cpu().numpy(), n_hist[3] - 1, hist, 64, W,
                               wl.n_kv_heads, wl.rope_base, wl.scale)
    tol_check(o1[3].double().cpu().numpy(), ref, torch.bfloat16, "attached seq 3")


def test_pool_exhaustion_and_block_reuse():
    W, Pmax, Bs = 64, 32, 16
    wl = configs.Workload("pge", torch.bfloat16, 2, 8, 4, 64, W, [16, 0], [1, 1], "decode")
    c = drive.make_cache(wl, prefix_max=Pmax, block_size=Bs, n_blocks=6, max_chunk=32)
    c.reset(0, 16)
    c.reset(1, 0)
    k, v = drive.kv_block(wl, [0, 0], 16 + W, "cuda")
    c.append(k, v, n_new=[16 + W, 0])         # 1 prefix block + 4 ring blocks
    table0, free = c.blocks(0)
    assert sum(t >= 0 for t in table0) == 5 and free == 1
    before = [c.export(s) for s in range(2)]
    k1, v1 = drive.kv_block(wl, [16 + W, 0], 32, "cuda")
    with pytest.raises(psa.PsaError) as e:       # sequence 1 needs 2 blocks, 1 is free
        c.append(k1, v1, n_new=[0, 32])
    assert e.value.status == psa.PSA_ERR_STATE
    with pytest.raises(psa.PsaError) as e:
        q = drive.query_block(wl, [16 + W, 0], 32, "cuda")
        c.prefill(q, k1, v1)
    assert e.value.status == psa.PSA_ERR_STATE
    assert c.seq_length(0) == 16 + W and c.seq_length(1) == 0
    assert c.blocks(0) == (table0, 1)
    after = [c.export(s) for s in range(2)]
    for x, y in zip(before, after):
        for a, b in zip(x, y):
            assert torch.equal(a, b)
    # one block is enough for 16 tokens; then resetting sequence 0 frees its 5 blocks,
    # which sequence 1 reuses (their stale contents must never be read)
    c.append(k1[:, :16].contiguous(), v1[:, :16].contiguous(), n_new=[0, 16])
    c.reset(0, 16)
    assert c.blocks(0)[1] == 5
    k2, v2 = drive.kv_block(wl, [0, 16], 200, "cuda")
    c.append(k2, v2, n_new=[0, 200])
    m = spec.WindowModel(0, W)
    for p in range(216):
        m.push(p)
    check_model(c, wl, 1, m)
    check_blocks(c, 2)
    table1, free = c.blocks(1)
    assert sum(t >= 0 for t in table1) == W // Bs and free == 6 - W // Bs
    c.promote(1, 20)                              # prefix slots 0 .. 19: two more blocks
    m.promote(20)
    assert c.blocks(1)[1] == 0
    check_model(c, wl, 1, m)
    with pytest.raises(psa.PsaError) as e:        # pool empty: no block for prefix slot 32
        k3, v3 = drive.kv_block(wl, [0, 0], 33, "cuda")
        c.append(k3, v3, n_new=[33, 0])
    assert e.value.status == psa.PSA_ERR_STATE
    kd, vd = drive.kv_block(wl, [0, 216], 1, "cuda")
    c.append(kd, vd, n_new=[0, 1])                # ring blocks are reused: no new block
    m.push(216)
    check_model(c, wl, 1, m)
    check_blocks(c, 2)


def test_paged_decode_full_size():
    # The 64-sequence decode shape (16/8 heads, D = 128, W = 4096, t = 32768) with a
    # 128-slot prefix region in 64-slot blocks: identical outputs to the contiguous cache.
    wl = configs.decode_p100_w4096()
    caches = [drive.make_cache(wl, prefix_max=128), drive.make_cache(wl, prefix_max=128, block_size=64)]
    n_hist = [wl.start[b] - 1 for b in range(wl.batch)]
    for c in caches:
        drive.fill(c, wl, n_hist)
    k, v = drive.kv_block(wl, n_hist, 1, "cuda")
    q = drive.queries(wl, n_hist, "cuda")
    outs = []
    for c in caches:
        c.append(k, v)
        lse = torch.empty((wl.batch, wl.n_q_heads), dtype=torch.float32, device="cuda")
        outs.append((c.decode(q, lse=lse), lse))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    check_blocks(caches[1], wl.batch)
    for s in (0, 37):
        np.testing.assert_array_equal(bits(caches[0].export(s)[0]), bits(caches[1].export(s)[0]))


@pytest.mark.parametrize("Hq,Hkv,D,dtype", [(32, 8, 128, torch.bfloat16), (64, 8, 128, torch.bfloat16),
                                            (16, 4, 64, torch.bfloat16), (8, 8, 64, torch.float32)])
def test_paged_decode_and_prefill_head_layouts(Hq, Hkv, D, dtype):
    # Every query-group size (G = 1, 4, 8) and head dimension has its own decode (and, for
    # bf16, prefill) instantiation; each must give the contiguous cache's exact results.
    W, Pmax, Bs = 256, 64, 32
    prefix = [30, 0, 64]
    n = [400, 100, 700]
    B = len(prefix)
    C = 48 if dtype == torch.bfloat16 else 0
    wl = configs.Workload("pgh", dtype, B, Hq, Hkv, D, W, prefix, [1] * B, "decode")
    caches = [drive.make_cache(wl, prefix_max=Pmax, max_chunk=C),
              drive.make_cache(wl, prefix_max=Pmax, max_chunk=C, block_size=Bs)]
    for c in caches:
        drive.fill(c, wl, n)
    if C:
        q = drive.query_block(wl, n, C, "cuda")
        k, v = drive.kv_block(wl, n, C, "cuda")
        o0, o1 = (c.prefill(q, k, v) for c in caches)
        assert torch.equal(o0, o1)
        n = [x + C for x in n]
    k, v = drive.kv_block(wl, n, 1, "cuda")
    q = drive.queries(wl, n, "cuda")
    outs = []
    for c in caches:
        c.append(k, v)
        outs.append(c.decode(q))
    assert torch.equal(outs[0], outs[1])
    same_export(caches[0], caches[1], B)
    check_blocks(caches[1], B)
    out = outs[1].double().cpu().numpy()
    qc = q.double().cpu().numpy()
    for s in range(B):
        ref, _ = attn.decode_query(qc[s], n[s], drive.hist_provider(wl, s), prefix[s], W, Hkv,
                                   wl.rope_base, wl.scale)
        tol_check(out[s], ref, dtype, f"seq {s}")
