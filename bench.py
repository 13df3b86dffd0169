"""Decode benchmark of prefix-pinned sliding-window attention on one MI355X.

A step is one pass of the decode hot path over the batch: append the new token of every
sequence (rotary encoding at its absolute position, ring write = eviction) and decode
attention for it (split-KV partials over the pinned prefix and the window, then the
cross-split merge). By default the step is one psa_decode_step call, whose decode launch
also performs the append; --step separate times psa_append then psa_decode_attn. Inputs for every step are generated before the timed region and are
resident in HBM when it starts; the state advances by one token per step.

Default workload: bf16, 64 sequences at t = 32768, 16 query / 8 KV heads, D = 128,
P = 100, W = 4096 (4196 visible positions per sequence).

Prints one JSON line with the throughput, the roofline of the dominant kernel (the
split-KV decode kernel, timed with HIP events on its launch stream in a separate pass)
and the float64 CPU oracle timed on a bounded sample of the same step.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode attn tokens/s + achieved HBM GB/s (% peak), bf16 GQA P=100 W=4096"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partial_traffic.json")
DECODE_SRC = os.path.join(ROOT, "prefix_pinned_sliding_amd", "csrc", "decode.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_p100_w4096",
                    choices=["decode_p100_w4096", "decode_p512_w16384", "ragged_decode",
                             "decode_shared_p2000", "decode_private_p2000",
                             "decode_ragged_window"])
    ap.add_argument("--t", type=int, default=0, help="override the start position t (flat-in-t sweeps)")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--block-size", type=int, default=0,
                    help="paged K/V in blocks of this many slots (0: contiguous); the prefix "
                         "region is rounded up to a multiple of it")
    ap.add_argument("--pe", default="continue", choices=["continue", "reset"],
                    help="position encoding of attended tokens (reset: renumber the cache list)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-calls", type=int, default=100)
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--train-calls", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other decode workloads and the flat-in-t sweep")
    ap.add_argument("--only", default="", choices=["", "prefill", "train"],
                    help="run only the chunked-prefill or the training benchmark and print its "
                         "JSON (for profiler runs of one kernel family)")
    ap.add_argument("--step", default="fused", choices=["fused", "separate"],
                    help="decode step as one psa_decode_step call (append + decode in one "
                         "launch) or as psa_append then psa_decode_attn")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB with torch (counter calibration)")
    return ap.parse_args()


def visible_entries(wl, n) -> int:
    """Cached entries a decode step reads: sum over sequences of min(n_b, P_b + w_b), the
    size of A(t) ([PS] 03) for histories of n_b tokens."""
    return sum(min(nb, pb + wl.window_of(b)) for b, (nb, pb) in enumerate(zip(n, wl.prefix)))


def source_hash(path: str) -> str:
    """Hash of a kernel source's code: // comments, surrounding blanks and empty lines are
    dropped, so the counter file stays tied to the code and not to its comments."""
    import re
    lines = []
    for line in open(path, encoding="utf-8"):
        code = re.sub(r"//.*", "", line).strip()
        if code:
            lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def load_traffic(launch_bytes_alg: float):
    """HBM bytes per decode launch from the committed counter runs, if they were taken on
    the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    if d.get("decode_code_sha256_16") != source_hash(DECODE_SRC):
        return None
    return d.get("hbm_bytes_per_launch")


_ORACLE_INPUTS = {}   # sequence -> (query position, visible positions, k, v) for the workers


def _oracle_worker(job):
    """Run the float64 oracle on sequences `seqs` of one decode step, round after round
    (at most 4), until `budget_s` seconds of oracle time; returns (queries, seconds). The
    inputs were generated by the parent before the fork; only the oracle call is timed."""
    wl, seqs, q_rows, budget_s = job
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attn

    def provider(key, k, v):
        def hist(req):
            assert np.asarray(req, dtype=np.int64).tobytes() == key
            return k, v
        return hist

    prepared = [(b, _ORACLE_INPUTS[b]) for b in seqs]
    done, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        for _ in range(4):
            for b, (p, pos, k32, v32) in prepared:
                hist = provider(pos.tobytes(), k32.astype(np.float64), v32.astype(np.float64))
                t0 = time.perf_counter()
                attn.decode_query(q_rows[b], p, hist, wl.prefix[b], wl.window_of(b),
                                  wl.n_kv_heads, wl.rope_base, wl.scale)
                elapsed += time.perf_counter() - t0
                done += 1
            if elapsed >= budget_s:
                break
    return done, elapsed


def cpu_baseline(wl, n_now, q_rows, budget_s: float):
    """The float64 oracle (as is) on the same decode step: the batch's sequences spread over
    worker processes, one per host core (at most 16, the GPU's share of the host), one BLAS
    thread each. Throughput = sum over workers of queries / oracle seconds. Inputs are
    generated first (not timed) and the workers are forked before the process touches the
    GPU. One worker alone gives the single-core figure."""
    import multiprocessing as mp

    import numpy as np

    from oracle import attn
    from synth import drive

    for b in range(wl.batch):
        p = n_now[b] - 1
        pos = np.nonzero(attn.visible_mask(wl.prefix[b], wl.window_of(b), p))[0]
        k, v = drive.hist_provider(wl, b)(pos)       # bf16 values: exact in float32
        _ORACLE_INPUTS[b] = (p, pos, k.astype(np.float32), v.astype(np.float32))
    n_cores = max(1, min(16, len(os.sched_getaffinity(0)), wl.batch))
    ctx = mp.get_context("fork")
    with ctx.Pool(1) as pool:
        one_done, one_s = pool.map(_oracle_worker, [(wl, [0, 1], q_rows, 2.0)])[0]
    jobs = [(wl, list(range(w, wl.batch, n_cores)), q_rows, budget_s) for w in range(n_cores)]
    with ctx.Pool(n_cores) as pool:
        res = pool.map(_oracle_worker, jobs)
    _ORACLE_INPUTS.clear()
    rate = sum(d / e for d, e in res)
    done = sum(d for d, _ in res)
    secs = max(e for _, e in res)
    return {"value": rate, "unit": "tokens/s", "cores": n_cores, "kind": "oracle",
            "single_core_value": one_done / one_s,
            "sample": f"the {wl.batch} sequences of one decode step (all {wl.n_q_heads} query "
                      f"heads, float64 NumPy, 1 BLAS thread per process) over {n_cores} "
                      f"processes: {done} queries, at most {secs:.1f} s of oracle time per "
                      f"process; single core: {one_done} queries in {one_s:.1f} s"}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_prefill(calls: int, warmup: int = 20):
    """Chunked prefill: 8 sequences each take a 512-token chunk at t ~ U{8192..65536}.

    Each call attends the chunk (staging, MFMA attention) and appends it; the state
    advances by 512 tokens per call. `warmup` untimed calls first bring the GPU to its
    steady clocks (a call takes about 0.2 ms), then `calls` timed ones and `calls` more with
    per-kernel events. Algorithmic work per call: 4 * H_q * D * sum over
    the chunk's queries of |A(p)| flops (QK^T and PV over the visible set).
    """
    import torch

    import prefix_pinned_sliding_amd as psa
    from synth import configs, drive

    wl = configs.prefill_chunk512()
    C = wl.chunk
    n0 = [t - 1 for t in wl.start]
    c = drive.make_cache(wl, max_chunk=C)
    drive.fill(c, wl, n0)
    total = warmup + 2 * calls
    inputs = []
    for i in range(total):
        starts = [n + i * C for n in n0]
        q = drive.query_block(wl, starts, C, "cuda")
        k, v = drive.kv_block(wl, starts, C, "cuda")
        inputs.append((q, k, v))
    out = torch.empty_like(inputs[0][0])
    torch.cuda.synchronize()
    for i in range(warmup):
        c.prefill(*inputs[i], out=out)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(warmup, warmup + calls):
        c.prefill(*inputs[i], out=out)
    stop.record()
    torch.cuda.synchronize()
    ms_call = start.elapsed_time(stop) / calls
    c.profile(True)
    for i in range(warmup + calls, total):
        c.prefill(*inputs[i], out=out)
    torch.cuda.synchronize()
    times = {name: c.profile_read(k) for k, name in psa.KERNEL_NAMES.items()}
    c.profile(False)
    pf_ms, pf_n = times["prefill"]
    pf_avg_s = pf_ms / pf_n / 1e3

    def visible(p, P):
        return min(p + 1, P + wl.window)

    flops = 0.0
    for i in range(warmup + calls, total):
        for b in range(wl.batch):
            base = n0[b] + i * C
            flops += sum(visible(base + j, wl.prefix[b]) for j in range(C))
    flops = flops / calls * 4 * wl.n_q_heads * wl.head_dim
    tflops = flops / pf_avg_s / 1e12
    return {"workload": wl.name, "calls": calls, "ms_per_call": ms_call,
            "tokens_per_s": wl.batch * C / (ms_call / 1e3),
            "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
                         "kernel": "prefill", "kernel_avg_us": pf_avg_s * 1e6,
                         "flops_per_launch": flops},
            "kernels_avg_us": {k: (ms / n * 1e3 if n else None) for k, (ms, n) in times.items()}}


def bench_train(calls: int, warmup: int = 2):
    """Training attention on the truncated back-propagation shape of the pages: a 100-token
    prompt plus 4W = 16384 lead tokens with W = 4096, 4 sequences, 16/8 heads, D = 128.

    Forward writes out and lse; backward computes dq, dk, dv from them. Algorithmic flops
    (the FlashAttention convention): forward 2 products, backward 5 (S recomputed, dP, dV,
    dK, dQ), each 2 * H_q * D * sum over rows of |A(row)| flops. Timed with events on the
    stream the kernels are launched on (torch's current stream).
    """
    import torch

    import prefix_pinned_sliding_amd as psa
    from synth import gen

    B, W, P, Hq, Hkv, D = 4, 4096, 100, 16, 8, 128
    T = P + 4 * W

    def draw(stream, H):
        return gen.normal_block(0, stream, list(range(B)), [0] * B, T, H, D, torch.bfloat16, "cuda")

    q, k, v, g = draw(gen.STREAM_Q, Hq), draw(gen.STREAM_K, Hkv), draw(gen.STREAM_V, Hkv), \
        draw(gen.STREAM_DO, Hq)
    ta = psa.TrainAttention(B, T, Hq, Hkv, D, W)
    pre = [P] * B
    out, lse = ta.forward(q, k, v, pre)
    dq, dk, dv = ta.backward(q, k, v, out, lse, g, pre)
    for _ in range(warmup):
        ta.forward(q, k, v, pre, out=out, lse=lse)
        ta.backward(q, k, v, out, lse, g, pre, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(calls):
        ta.forward(q, k, v, pre, out=out, lse=lse)
    ev[1].record()
    for _ in range(calls):
        ta.backward(q, k, v, out, lse, g, pre, dq=dq, dk=dk, dv=dv)
    ev[2].record()
    torch.cuda.synchronize()
    fwd_s = ev[0].elapsed_time(ev[1]) / calls / 1e3
    bwd_s = ev[1].elapsed_time(ev[2]) / calls / 1e3
    pairs = sum(i + 1 if i < P else P + min(W, i - P + 1) for i in range(T)) * B
    unit = 2.0 * Hq * D * pairs
    fwd_tf, bwd_tf = 2 * unit / fwd_s / 1e12, 5 * unit / bwd_s / 1e12
    return {"workload": f"train-bf16-B{B}-P{P}-W{W}-T{T}", "calls": calls,
            "fwd_ms": fwd_s * 1e3, "bwd_ms": bwd_s * 1e3,
            "tokens_per_s_fwd_bwd": B * T / (fwd_s + bwd_s),
            "fwd_tflops": fwd_tf,
            "roofline": {"bound": "mfma", "achieved": bwd_tf, "peak": MFMA_BF16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": bwd_tf / MFMA_BF16_PEAK_TFLOPS,
                         "kernel": "backward (rowdot + dkdv + dq)", "flops_per_launch": 5 * unit}}


def fill_timing(cache, wl, n_hist, block=4096) -> None:
    """Bring every sequence to n_hist[b] tokens through real appends (eviction included),
    with one seeded [B][block][H_kv][D] block of values appended over and over: the
    timing-only sweeps read the same visible set whatever the values, and drawing every
    position of a 131072-token history would dominate the run."""
    import torch

    from synth import drive

    B = wl.batch
    for b in range(B):
        cache.reset(b, wl.prefix[b])
        if wl.windows is not None:
            cache.set_window(b, wl.windows[b])
    k, v = drive.kv_block(wl, [0] * B, block, "cuda")
    done = [0] * B
    while any(d < n for d, n in zip(done, n_hist)):
        counts = [min(block, n - d) for d, n in zip(done, n_hist)]
        cache.append(k, v, n_new=counts)
        done = [d + c for d, c in zip(done, counts)]
    torch.cuda.synchronize()


def time_steps(c, wl, n0, warmup: int, steps: int, fused: bool = True):
    """warmup + steps decode steps from histories n0 (the state advances one token per
    step), the timed steps between two events; then `steps` more with per-kernel events.
    Returns (ms per step, {kernel: (total ms, launches)}, visible entries of the first and
    last profiled step)."""
    import torch

    import prefix_pinned_sliding_amd as psa
    from synth import drive

    total = warmup + 2 * steps
    ks, vs, qs = [], [], []
    for i in range(total):
        k, v = drive.kv_block(wl, [n + i for n in n0], 1, "cuda")
        ks.append(k[:, 0].contiguous() if fused else k)
        vs.append(v[:, 0].contiguous() if fused else v)
        qs.append(drive.queries(wl, [n + i for n in n0], "cuda"))
    out = torch.empty_like(qs[0])

    def step(i):
        if fused:
            c.decode_step(ks[i], vs[i], qs[i], out)
        else:
            c.append(ks[i], vs[i])
            c.decode(qs[i], out)

    c.decode(qs[0], out)     # untimed: loads the kernels, only reads the cache
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(warmup, warmup + steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    c.profile(True)
    for i in range(warmup + steps, total):
        step(i)
    torch.cuda.synchronize()
    times = {name: c.profile_read(k) for k, name in psa.KERNEL_NAMES.items()}
    c.profile(False)
    vis = (visible_entries(wl, [n + warmup + steps + 1 for n in n0]),
           visible_entries(wl, [n + total for n in n0]))
    return ms, times, vis


def decode_roofline(wl, times, vis):
    elem = 2 if str(wl.dtype) == "torch.bfloat16" else 4
    dec_ms, dec_n = times["decode_partial"]
    dec_s = dec_ms / dec_n / 1e3
    launch_bytes = 0.5 * (vis[0] + vis[1]) * wl.n_kv_heads * wl.head_dim * 2 * elem
    achieved = launch_bytes / dec_s / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "kernel": "decode_partial",
            "kernel_avg_us": dec_s * 1e6, "bytes_per_launch": launch_bytes}


def bench_decode_config(name: str, warmup: int, steps: int):
    """Another decode workload's fused step: µs per step, tokens/s and the decode kernel's
    roofline. Histories are filled with real seeded values (drive.fill)."""
    import torch

    from synth import configs, drive

    wl = configs.by_name(name)
    n0 = [t - 1 for t in wl.start]
    c = drive.make_cache(wl)
    drive.fill(c, wl, n0)
    ms, times, vis = time_steps(c, wl, n0, warmup, steps)
    del c
    torch.cuda.empty_cache()
    return {"workload": wl.name, "warmup": warmup, "steps": steps, "ms_per_step": ms,
            "tokens_per_s": wl.batch / (ms / 1e3),
            "visible_tokens_per_step": 0.5 * (vis[0] + vis[1]),
            "roofline": decode_roofline(wl, times, vis),
            "kernels_avg_us": {k: (t / n * 1e3 if n else None) for k, (t, n) in times.items()}}


FLAT_T = (2148, 4196, 8392, 32768, 131072)


def bench_flat_in_t(warmup: int = 10, steps: int = 50, rounds: int = 3):
    """The default decode shape (64 sequences, P = 100, W = 4096) at several t: the step
    must cost the same once the window is full ([PS] 04: per-step cost O((P + W) d),
    independent of t). Each t has its own cache, reset and filled by appends; the t values
    are timed in interleaved rounds (t1, t2, ..., t1, t2, ...), so that a change of clock
    during the sweep falls on every t alike, and each t reports the median of its rounds."""
    import torch

    from synth import configs, drive

    wl = configs.decode_p100_w4096()
    B = wl.batch
    state = {}
    for t in FLAT_T:
        c = drive.make_cache(wl)
        fill_timing(c, wl, [t - 1] * B)
        state[t] = [c, t - 1]
    runs = {t: [] for t in FLAT_T}
    for _ in range(rounds):
        for t in FLAT_T:
            c, n = state[t]
            ms, times, vis = time_steps(c, wl, [n] * B, warmup, steps)
            state[t][1] = n + warmup + 2 * steps
            runs[t].append((ms * 1e3, times["decode_partial"][0] / times["decode_partial"][1] * 1e3,
                            vis[1] // B))
    del state, c
    torch.cuda.empty_cache()
    res = {}
    for t in FLAT_T:
        step_us = sorted(r[0] for r in runs[t])
        part_us = sorted(r[1] for r in runs[t])
        res[str(t)] = {"us_per_step": step_us[len(step_us) // 2],
                       "decode_partial_us": part_us[len(part_us) // 2],
                       "us_per_step_rounds": [r[0] for r in runs[t]],
                       "visible_per_sequence": runs[t][-1][2]}
    full = [res[str(t)]["us_per_step"] for t in FLAT_T if t >= 4196]
    return {"workload": "decode-bf16-B64-P100-W4096 at several t", "warmup": warmup,
            "steps": steps, "rounds": rounds, "t": res,
            "spread_full_window": (max(full) - min(full)) / (sum(full) / len(full))}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(run one process per GPU; sequences and KV heads shard with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from synth import configs, drive, gen

    if args.only:
        torch.cuda.set_device(0)
        res = bench_prefill(args.prefill_calls) if args.only == "prefill" else \
            bench_train(args.train_calls)
        print(json.dumps({args.only: res}), flush=True)
        return

    if args.workload == "decode_p100_w4096":
        wl = configs.decode_p100_w4096(t=args.t) if args.t else configs.decode_p100_w4096()
    elif args.workload == "decode_p512_w16384":
        wl = configs.decode_p512_w16384(t=args.t) if args.t else configs.decode_p512_w16384()
    elif args.workload in ("decode_shared_p2000", "decode_private_p2000"):
        wl = configs.decode_shared_p2000(t=args.t) if args.t else configs.decode_shared_p2000()
        if args.workload == "decode_private_p2000":
            wl.name = wl.name.replace("shared", "private")
    elif args.workload == "decode_ragged_window":
        wl = configs.decode_ragged_window(t=args.t) if args.t else configs.decode_ragged_window()
    else:
        wl = configs.ragged_decode()
    B = wl.batch
    n0 = [t - 1 for t in wl.start]
    total = args.warmup + 2 * args.steps
    n_prof = [n + total for n in n0]          # history length during the last profiled step

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle on the last profiled step's queries, before the GPU is initialised
        print("[bench] cpu baseline (float64 oracle)", file=sys.stderr, flush=True)
        qc = drive.queries(wl, [n - 1 for n in n_prof], "cpu").double().numpy()
        cpu = cpu_baseline(wl, n_prof, qc, args.cpu_seconds)

    import prefix_pinned_sliding_amd as psa

    torch.cuda.set_device(0)
    print(f"[bench] {wl.name}: filling {sum(n0)} tokens", file=sys.stderr, flush=True)
    bs = args.block_size
    if args.workload == "decode_shared_p2000":
        c = drive.make_cache(wl, n_shared=1, shared_max=wl.prefix[0], prefix_max=0, pe=args.pe,
                             block_size=bs)
    else:
        pmax = -(-wl.prefix_max // bs) * bs if bs else wl.prefix_max
        c = drive.make_cache(wl, pe=args.pe, prefix_max=pmax, block_size=bs)
    if args.split_tokens:
        c.set_split_tokens(args.split_tokens)
    if args.workload in ("decode_shared_p2000", "decode_private_p2000"):
        drive.fill_one_prompt(c, wl, n0, shared=args.workload == "decode_shared_p2000")
    else:
        drive.fill(c, wl, n0)

    # inputs of every step, resident before timing
    ks, vs, qs = [], [], []
    for i in range(total):
        k, v = drive.kv_block(wl, [n + i for n in n0], 1, "cuda")
        ks.append(k)
        vs.append(v)
        qs.append(drive.queries(wl, [n + i for n in n0], "cuda"))
    out = torch.empty_like(qs[0])
    torch.cuda.synchronize()
    print(f"[bench] inputs ready; {args.warmup} warmup + {args.steps} timed steps", file=sys.stderr,
          flush=True)

    if args.step == "fused":
        ks = [k[:, 0] for k in ks]                 # [B][H_kv][D] views (contiguous)
        vs = [v[:, 0] for v in vs]

        def step(i):
            c.decode_step(ks[i], vs[i], qs[i], out)
    else:
        def step(i):
            c.append(ks[i], vs[i])
            c.decode(qs[i], out)

    # One untimed decode on the filled state loads the decode kernels (decode only reads
    # the cache, so the state the steps start from is unchanged; ragged_decode runs
    # without warmup steps to keep its 64 states).
    c.decode(qs[0], out)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    stop.record()
    torch.cuda.synchronize()
    ms_total = start.elapsed_time(stop)
    ms_per_step = ms_total / args.steps
    print(f"[bench] timed: {ms_per_step * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    # second pass: per-kernel HIP events around each launch on the launch stream
    c.profile(True)
    for i in range(args.warmup + args.steps, total):
        step(i)
    torch.cuda.synchronize()
    times = {name: c.profile_read(k) for k, name in psa.KERNEL_NAMES.items()}
    c.profile(False)
    dec_ms, dec_n = times["decode_partial"]
    dec_avg_s = dec_ms / dec_n / 1e3

    # algorithmic bytes of one decode launch: the visible K and V rows of every sequence
    elem = 2 if wl.dtype == torch.bfloat16 else 4
    vis_first = visible_entries(wl, [n + args.warmup + args.steps + 1 for n in n0])
    vis_last = visible_entries(wl, n_prof)
    vis = 0.5 * (vis_first + vis_last)
    launch_bytes = vis * wl.n_kv_heads * wl.head_dim * 2 * elem
    achieved = launch_bytes / dec_avg_s / 1e9
    traffic = load_traffic(launch_bytes) if (args.workload == "decode_p100_w4096" and not bs
                                             and args.pe == "continue" and not args.t) else None

    result = {
        "metric": METRIC,
        "value": B / (ms_per_step / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "q_heads": wl.n_q_heads,
                   "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "prefix": wl.prefix[0] if len(set(wl.prefix)) == 1 else "ragged",
                   "window": wl.window if wl.windows is None else "ragged",
                   "t": wl.start[0] if len(set(wl.start)) == 1 else "ragged",
                   "visible_tokens_per_step": vis, "parallelism": "single GPU",
                   "position_encoding": args.pe, "kv_block_size": bs, "step_calls": args.step},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel": "decode_partial",
                     "kernel_avg_us": dec_avg_s * 1e6, "bytes_per_launch": launch_bytes},
        "kernels_avg_us": {k: (ms / n * 1e3 if n else None) for k, (ms, n) in times.items()},
    }
    # Decode attention alone (partial + merge) re-timed on the last state: 100 calls, each
    # between two HIP events on the launch stream; decode only reads the cache.
    rep = []
    for _ in range(100):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        c.decode(qs[total - 1], out)
        e1.record()
        rep.append((e0, e1))
    torch.cuda.synchronize()
    rep_us = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in rep)
    result["decode_repeat_us"] = {"median": rep_us[len(rep_us) // 2], "min": rep_us[0],
                                  "max": rep_us[-1], "repeats": len(rep_us)}
    mer_ms, mer_n = times["merge"]
    result["attention_only_tokens_per_s"] = B / (dec_avg_s + mer_ms / mer_n / 1e3)
    if bs:
        free = c.blocks(0)[1]
        total_blocks = c.layout.n_blocks
        result["paged"] = {"block_size": bs, "blocks_total": total_blocks,
                           "blocks_used": total_blocks - free,
                           "kv_bytes_used": (total_blocks - free) * bs * wl.n_kv_heads * wl.head_dim * 2 * elem}
    if traffic is not None:
        result["roofline"]["traffic_over_algorithmic"] = traffic / launch_bytes

    if not args.no_prefill and args.workload == "decode_p100_w4096":
        del c
        torch.cuda.empty_cache()
        print("[bench] chunked prefill", file=sys.stderr, flush=True)
        result["prefill"] = bench_prefill(args.prefill_calls)

    if not args.no_train and args.workload == "decode_p100_w4096":
        torch.cuda.empty_cache()
        print("[bench] training attention", file=sys.stderr, flush=True)
        result["train"] = bench_train(args.train_calls)

    if not args.no_extra and args.workload == "decode_p100_w4096" and not args.t:
        torch.cuda.empty_cache()
        print("[bench] decode P=512 W=16384", file=sys.stderr, flush=True)
        result["decode_p512_w16384"] = bench_decode_config("decode_p512_w16384", 10, 50)
        print("[bench] ragged decode B=256", file=sys.stderr, flush=True)
        result["ragged_decode"] = bench_decode_config("ragged_decode", 0, 64)
        print("[bench] decode with a window length per sequence", file=sys.stderr, flush=True)
        result["decode_ragged_window"] = bench_decode_config("decode_ragged_window", 10, 50)
        print("[bench] flat in t", file=sys.stderr, flush=True)
        result["flat_in_t"] = bench_flat_in_t()

    if cpu is not None:
        result["cpu_baseline"] = cpu

    if args.copy_probe_mib:
        nb = args.copy_probe_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: 3 x {nb} bytes", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
