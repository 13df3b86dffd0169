"""The host process pool that runs the oracle for the full-size GPU tests: a job gives the
same result as calling the oracle directly (CPU only)."""
import numpy as np
import torch

import oracle_pool as op
from oracle import attn, cache as ocache, rne
from synth import configs, drive


def small():
    return configs.Workload("pool", torch.bfloat16, 3, 8, 4, 64, 40, [7, 0, 30], [1, 1, 1],
                            "decode")


def test_decode_job_equals_direct_oracle_calls():
    wl = small()
    b, positions = 2, np.array([5, 29, 30, 75, 200])
    q = np.stack([drive.queries(wl, [p] * 3)[b].double().numpy() for p in positions])
    out, lse = op.decode_job((wl, b, positions, q, None))
    for i, p in enumerate(positions):
        ro, rl = attn.decode_query(q[i], int(p), drive.hist_provider(wl, b), 30, 40, 4,
                                   wl.rope_base, wl.scale)
        np.testing.assert_array_equal(out[i], ro)
        np.testing.assert_array_equal(lse[i], rl)


def test_composite_prefix_job():
    wl = small()
    q = drive.queries(wl, [90] * 3)[1:2].double().numpy()
    out, _ = op.decode_job((wl, 1, np.array([90]), q, 0))
    hist = drive.composite_history(wl, 0, 1, wl.prefix[1])
    ro, _ = attn.decode_query(q[0], 90, hist, wl.prefix[1], 40, 4, wl.rope_base, wl.scale)
    np.testing.assert_array_equal(out[0], ro)


def test_expected_view_digest_and_pool():
    wl = small()
    jobs = [(wl, b, n, "bf16") for b, n in [(0, 5), (0, 100), (2, 31)]]
    got = op.run(op.expected_view_job, jobs, workers=2)
    for (wl_, b, n, _), (cnt, dig) in zip(jobs, got):
        pos, kbits, vref = ocache.expected_view(wl.prefix[b], 40, n, drive.hist_provider(wl, b),
                                                wl.rope_base, "bf16")
        assert cnt == len(pos) == min(n, wl.prefix[b] + 40)
        assert dig == op.view_digest(pos, kbits, rne.f64_to_bf16_bits(vref))
    # any changed bit changes the digest
    pos, kbits, vref = ocache.expected_view(7, 40, 100, drive.hist_provider(wl, 0), wl.rope_base,
                                            "bf16")
    vb = rne.f64_to_bf16_bits(vref)
    kb2 = kbits.copy()
    kb2[3, 1, 5] ^= 1
    assert op.view_digest(pos, kb2, vb) != got[1][1]


def test_whole_tensor_error():
    ref = np.ones((2, 3, 4))
    out = ref.copy()
    out[1, 2, 3] += 0.5
    err, rel = op.whole_tensor_error(out, ref)
    assert err == 0.5 and abs(rel - 0.5 / np.sqrt(24)) < 1e-15
