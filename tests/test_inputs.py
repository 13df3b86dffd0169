"""The seeded input generator: SplitMix64 against its published outputs, random access
by position, and the N(0,1) shape of the values."""
import json
import os

import numpy as np
import torch

from synth import configs, gen


def test_splitmix64_published_outputs(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "splitmix64_seed0.json")))
    gamma = 0x9E3779B97F4A7C15
    for i, h in enumerate(g["outputs_hex"], start=1):
        assert gen.mix_int(gamma * i) == int(h, 16)
    z = torch.tensor([gen._i64((gamma * i) % (1 << 64)) for i in range(1, 4)], dtype=torch.int64)
    got = [int(x) % (1 << 64) for x in gen.mix(z).tolist()]
    assert got == [int(h, 16) for h in g["outputs_hex"]]


def test_torch_mix_matches_integer_mix():
    rng = np.random.default_rng(0)
    vals = [int(x) for x in rng.integers(0, 1 << 63, 1000, dtype=np.uint64)] + [0, (1 << 64) - 1, 1 << 63]
    z = torch.tensor([gen._i64(v) for v in vals], dtype=torch.int64)
    got = [int(x) % (1 << 64) for x in gen.mix(z).tolist()]
    assert got == [gen.mix_int(v) for v in vals]


def test_random_access_by_position():
    a = gen.normal_rows(0, gen.STREAM_K, 5, 0, 300, 2, 16, torch.bfloat16)
    b = gen.normal_block(0, gen.STREAM_K, [5, 6], [100, 0], 50, 2, 16, torch.bfloat16)
    assert torch.equal(a[100:150], b[0])
    c = gen.normal_rows(0, gen.STREAM_K, 6, 0, 50, 2, 16, torch.bfloat16)
    assert torch.equal(b[1], c)
    assert not torch.equal(b[1], a[:50])


def test_streams_and_seeds_differ():
    a = gen.normal_rows(0, gen.STREAM_K, 0, 0, 64, 1, 64)
    b = gen.normal_rows(0, gen.STREAM_V, 0, 0, 64, 1, 64)
    c = gen.normal_rows(1, gen.STREAM_K, 0, 0, 64, 1, 64)
    assert not torch.equal(a, b) and not torch.equal(a, c)


def test_values_look_standard_normal():
    x = gen.normal_rows(0, gen.STREAM_Q, 3, 0, 2000, 8, 128, torch.float64).flatten().numpy()
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    assert abs(np.mean(np.abs(x) > 1.96) - 0.05) < 2e-3


def test_workload_draws_are_seeded_and_in_range():
    w = configs.ragged_decode()
    assert w == configs.ragged_decode()
    assert all(50 <= p <= 2000 for p in w.prefix)
    assert all(1000 <= t <= 131072 for t in w.start)
    pre = configs.prefill_chunk512()
    assert all(8192 <= t <= 65536 for t in pre.start)
    d = configs.decode_p100_w4096()
    assert (d.batch, d.window, d.prefix[0], d.start[0]) == (64, 4096, 100, 32768)
