"""The C-ABI library loads without a GPU, exports every function include/psa.h declares,
and rejects invalid arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "psa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(psa_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def psa():
    import prefix_pinned_sliding_amd as m
    return m


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["psa_cache_bytes", "psa_cache_create", "psa_cache_destroy", "psa_seq_reset",
                 "psa_append", "psa_decode_attn", "psa_decode_step", "psa_prefill_attn", "psa_export",
                 "psa_seq_length", "psa_status_string", "psa_last_error"]:
        assert want in names


def test_every_declared_symbol_is_exported(psa):
    raw = ctypes.CDLL(psa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_exports_only_the_c_abi(psa):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", psa.LIB_PATH], capture_output=True,
                         text=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert {s for s in syms if s.startswith("psa_")} == set(declared_functions())


def good_desc(psa, **kw):
    d = dict(max_batch=4, n_q_heads=16, n_kv_heads=8, head_dim=128, prefix_max=100, window=4096,
             max_chunk=512)
    d.update(kw)
    return psa.make_desc(**d)


def test_cache_bytes_and_layout(psa):
    d = good_desc(psa)
    n = psa.cache_bytes(d)
    L = psa.cache_layout(d)
    assert L.total_bytes == n
    S = 100 + 4096
    assert L.slots == S and L.elem_bytes == 2
    kv = 4 * 8 * S * 128 * 2
    assert L.v_offset >= L.k_offset + kv and L.tags_offset >= L.v_offset + kv
    for off in (L.k_offset, L.v_offset, L.tags_offset, L.state_offset, L.work_offset):
        assert off % 256 == 0
    assert n >= 2 * kv + 4 * S * 4


@pytest.mark.parametrize("bad", [
    dict(max_batch=0), dict(n_kv_heads=0), dict(n_q_heads=12), dict(n_q_heads=48, n_kv_heads=4),
    dict(head_dim=96), dict(prefix_max=-1), dict(window=0), dict(max_chunk=-1),
])
def test_invalid_descriptions_are_rejected(psa, bad):
    d = good_desc(psa, **bad)
    assert psa.lib.psa_cache_bytes(ctypes.byref(d)) == 0
    out = psa.Layout()
    assert psa.lib.psa_cache_layout(ctypes.byref(d), ctypes.byref(out)) == psa.PSA_ERR_ARG
    assert psa.lib.psa_last_error().decode() != ""


def test_invalid_rope_base_scale_dtype(psa):
    for field, val in [("rope_base", 0.0), ("rope_base", float("inf")), ("scale", -1.0),
                       ("dtype", 7), ("n_blocks", 1)]:
        d = good_desc(psa)
        setattr(d, field, val)
        assert psa.lib.psa_cache_bytes(ctypes.byref(d)) == 0, field


@pytest.mark.parametrize("bad", [
    dict(max_batch=65536), dict(n_q_heads=65536 * 2, n_kv_heads=65536),
    dict(window=1 << 24),                                        # prefill ring rows need < 2^24
    dict(max_chunk=(1 << 32) // (8 * 128)),                      # chunk rows x H_kv x D >= 2^32
])
def test_shapes_beyond_the_kernels_addressing_are_rejected(psa, bad):
    d = good_desc(psa, prefix_max=0, **bad)
    assert psa.lib.psa_cache_bytes(ctypes.byref(d)) == 0, bad
    assert psa.lib.psa_last_error().decode() != ""


def test_decode_grid_bound(psa):
    # the decode grid's x dimension holds n_kv_heads * splits workgroups of 256 threads:
    # n_kv_heads * (ceil(seen / 128) + 1) must stay below 2^24
    ok = good_desc(psa, max_batch=1, n_q_heads=1, n_kv_heads=1, prefix_max=0, window=1 << 28,
                   max_chunk=0)
    assert psa.cache_layout(ok).max_splits == (1 << 21) + 1
    d = good_desc(psa, max_batch=1, n_q_heads=8, n_kv_heads=8, prefix_max=0, window=1 << 28,
                  max_chunk=0)
    assert psa.lib.psa_cache_bytes(ctypes.byref(d)) == 0
    assert "decode splits" in psa.lib.psa_last_error().decode()
    # just inside: 8 * (2^21 - 2 + 1) < 2^24
    edge = good_desc(psa, max_batch=1, n_q_heads=8, n_kv_heads=8, prefix_max=0,
                     window=((1 << 21) - 2) * 128, max_chunk=0)
    assert psa.cache_layout(edge).max_splits == (1 << 21) - 1


def test_long_window_is_accepted_without_prefill(psa):
    # the 24-bit row bound belongs to chunked prefill only
    d = good_desc(psa, max_batch=1, n_q_heads=8, n_kv_heads=8, prefix_max=0, window=1 << 24,
                  max_chunk=0)
    assert psa.cache_layout(d).slots == 1 << 24
    assert psa.cache_layout(good_desc(psa, max_chunk=(1 << 32) // (8 * 128) - 1)).slots == 4196


def test_split_slots_cover_shared_prefixes(psa):
    # an attached sequence sees up to shared_prefix_max + window entries, more than
    # prefix_max + window: the decode workspace must hold the splits of that many
    d = good_desc(psa, prefix_max=0, window=128, n_shared_prefixes=1, shared_prefix_max=512,
                  max_chunk=0)
    L = psa.cache_layout(d)
    assert L.max_splits >= -(-(512 + 128) // 128)          # 5 splits of 128 entries
    assert psa.cache_layout(good_desc(psa)).max_splits >= -(-(100 + 4096) // 128)
    # RESET cuts the prefix and the window separately: one more split
    r = psa.cache_layout(good_desc(psa, pe="reset"))
    assert r.max_splits >= -(-100 // 128) + -(-4096 // 128)


def test_paged_layout(psa):
    # K/V become a pool of blocks [H_kv][n_blocks][Bs][D]; the block table follows the tags
    d = good_desc(psa, prefix_max=128, block_size=64)
    L = psa.cache_layout(d)
    S = 128 + 4096
    assert L.slots == S and L.block_size == 64 and L.n_blocks == 4 * S // 64
    kv = L.n_blocks * 8 * 64 * 128 * 2
    assert L.v_offset >= L.k_offset + kv and L.tags_offset >= L.v_offset + kv
    assert L.btab_offset >= L.tags_offset + 4 * S * 4
    assert L.state_offset >= L.btab_offset + 4 * (S // 64) * 4
    for off in (L.btab_offset, L.state_offset):
        assert off % 256 == 0
    # a smaller pool shrinks the K/V regions only
    small = psa.cache_layout(good_desc(psa, prefix_max=128, block_size=64, n_blocks=10))
    assert small.n_blocks == 10
    assert L.total_bytes - small.total_bytes == 2 * (L.n_blocks - 10) * 8 * 64 * 128 * 2


@pytest.mark.parametrize("bad", [
    dict(block_size=48), dict(block_size=8), dict(block_size=64),          # 100 % 64 != 0
    dict(prefix_max=128, block_size=64, n_blocks=-1),
    dict(prefix_max=0, window=65536, block_size=16),                      # table > 1024 entries
    dict(n_blocks=5),                                                      # contiguous with a pool
])
def test_invalid_paged_descriptions(psa, bad):
    d = good_desc(psa, **bad)
    assert psa.lib.psa_cache_bytes(ctypes.byref(d)) == 0, bad
    assert psa.lib.psa_last_error().decode() != ""


def test_seq_blocks_needs_a_handle(psa):
    n = ctypes.c_int32()
    assert psa.lib.psa_seq_blocks(None, 0, None, ctypes.byref(n), None) == psa.PSA_ERR_ARG


def test_create_rejects_bad_buffers_before_any_device_call(psa):
    d = good_desc(psa)
    n = psa.cache_bytes(d)
    h = ctypes.c_void_p()
    lib = psa.lib
    assert lib.psa_cache_create(ctypes.byref(d), None, n, None, ctypes.byref(h)) == psa.PSA_ERR_ARG
    assert lib.psa_cache_create(ctypes.byref(d), ctypes.c_void_p(0x1000 + 8), n, None,
                                ctypes.byref(h)) == psa.PSA_ERR_ARG
    assert "aligned" in lib.psa_last_error().decode()
    assert lib.psa_cache_create(ctypes.byref(d), ctypes.c_void_p(0x100000), n - 1, None,
                                ctypes.byref(h)) == psa.PSA_ERR_ARG
    assert "too small" in lib.psa_last_error().decode()
    assert h.value is None


def test_null_handle_calls(psa):
    lib = psa.lib
    assert lib.psa_cache_destroy(None) == psa.PSA_OK
    assert lib.psa_seq_reset(None, 0, 0, None) == psa.PSA_ERR_ARG
    assert lib.psa_append(None, None, 1, None, None, 1, None) == psa.PSA_ERR_ARG
    assert lib.psa_decode_attn(None, None, None, None, None) == psa.PSA_ERR_ARG
    assert lib.psa_decode_step(None, None, None, None, None, None, None) == psa.PSA_ERR_ARG
    assert lib.psa_prefill_attn(None, 1, None, None, None, None, None, None) == psa.PSA_ERR_ARG
    cnt = ctypes.c_int32()
    assert lib.psa_export(None, 0, None, None, None, ctypes.byref(cnt), None) == psa.PSA_ERR_ARG
    assert lib.psa_seq_length(None, 0) == -1
    assert lib.psa_set_split_tokens(None, 0) == psa.PSA_ERR_ARG


def test_status_strings(psa):
    for s in range(5):
        assert psa.lib.psa_status_string(s).decode()
    assert psa.lib.psa_status_string(99).decode() == "unknown status"


def test_train_workspace_and_validation(psa):
    lib = psa.lib
    d = psa.TrainDesc(4, 1000, 16, 8, 128, 256, 0.0, 0)
    n = lib.psa_train_workspace_bytes(ctypes.byref(d))
    assert n >= 4 * 1000 * 16 * 4 and n % 256 == 0       # float32 Di per (row, head)
    for bad in [psa.TrainDesc(0, 1000, 16, 8, 128, 256, 0.0, 0),
                psa.TrainDesc(4, 0, 16, 8, 128, 256, 0.0, 0),
                psa.TrainDesc(4, 1000, 12, 8, 128, 256, 0.0, 0),
                psa.TrainDesc(4, 1000, 48, 3, 128, 256, 0.0, 0),
                psa.TrainDesc(4, 1000, 16, 8, 96, 256, 0.0, 0),
                psa.TrainDesc(4, 1000, 16, 8, 128, 0, 0.0, 0),
                psa.TrainDesc(4, 1000, 16, 8, 128, 256, -1.0, 0),
                psa.TrainDesc(4, 1000, 16, 8, 128, 256, 0.0, 7)]:
        assert lib.psa_train_workspace_bytes(ctypes.byref(bad)) == 0
        assert lib.psa_last_error()
    # null pointers are rejected on the host (nothing reaches the device)
    pre = (ctypes.c_int32 * 4)(0, 0, 0, 0)
    rc = lib.psa_train_fwd(ctypes.byref(d), pre, None, None, None, None, None, None, None, 0, None)
    assert rc == psa.PSA_ERR_ARG


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_import_fails_loudly_without_the_library(tmp_path):
    # the binding has no fallback: a package tree without libpsa.so must not import
    import shutil
    import subprocess
    import sys
    pkg = tmp_path / "prefix_pinned_sliding_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "prefix_pinned_sliding_amd", "__init__.py"), pkg / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import prefix_pinned_sliding_amd"],
                       cwd=str(tmp_path), capture_output=True, text=True, timeout=120,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "libpsa.so" in r.stderr


def test_counter_file_is_tied_to_kernel_code_not_comments(tmp_path):
    # bench.py reports HBM traffic only while the decode kernel's code is the one the
    # counters were taken on; a comment edit keeps the hash, a code edit changes it
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    src = open(bench.DECODE_SRC).read()
    a, b, c = tmp_path / "a.hip", tmp_path / "b.hip", tmp_path / "c.hip"
    a.write_text(src)
    b.write_text("// a new comment\n" + src.replace("\n", "  // note\n", 3) + "\n\n")
    c.write_text(src.replace("kRescaleSlack = 8.0f", "kRescaleSlack = 7.0f"))
    assert bench.source_hash(str(a)) == bench.source_hash(str(b))
    assert bench.source_hash(str(a)) != bench.source_hash(str(c))


def test_noalloc_backward_rejects_shapes_beyond_its_static_scratch(psa):
    # B * T * H_q float32 row dots above PSA_TRAIN_STATIC_SCRATCH_BYTES: refused on the host,
    # before any device call (the pointers are never touched)
    d = psa.TrainDesc(1, 1 << 20, 8, 8, 128, 4096, 0.0, 0)
    assert psa.lib.psa_train_workspace_bytes(ctypes.byref(d)) > 16 << 20
    pre = (ctypes.c_int32 * 1)(0)
    fake = [ctypes.c_void_p(0x1000 * (i + 1)) for i in range(9)]
    rc = psa.lib.psa_train_bwd_noalloc(ctypes.byref(d), pre, None, *fake, None)
    assert rc == psa.PSA_ERR_ARG
    assert "static scratch" in psa.lib.psa_last_error().decode()
    d.n_q_heads = 12          # and the ordinary shape checks still come first
    assert psa.lib.psa_train_bwd_noalloc(ctypes.byref(d), pre, None, *fake, None) == psa.PSA_ERR_ARG
