"""Decode benchmark of prefix-pinned sliding-window attention on one MI355X.

A step is one pass of the decode hot path over the batch: append the new token of every
sequence (rotary encoding at its absolute position, ring write = eviction) and decode
attention for it (split-KV partials over the pinned prefix and the window, then the
cross-split merge). Inputs for every step are generated before the timed region and are
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
    ap.add_argument("--pe", default="continue", choices=["continue", "reset"],
                    help="position encoding of attended tokens (reset: renumber the cache list)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-calls", type=int, default=10)
    ap.add_argument("--no-train", action="store_true")
    ap.add_argument("--train-calls", type=int, default=5)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the run, copy this many MiB with torch (counter calibration)")
    return ap.parse_args()


def source_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def load_traffic(launch_bytes_alg: float):
    """HBM bytes per decode launch from the committed counter runs, if they were taken on
    the current kernel source; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    if d.get("decode_src_sha256_16") != source_hash(DECODE_SRC):
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(wl, n_now, q_rows, budget_s: float):
    """Time the float64 oracle (as is) on a bounded sample of the step's sequences.

    Inputs (the visible K/V rows) are generated first and are not timed. BLAS is held to
    one thread, so the oracle runs on one core.
    """
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import attn
    from synth import drive

    def prepared(b):
        full = drive.hist_provider(wl, b)
        p = n_now[b] - 1
        pos = np.nonzero(attn.visible_mask(wl.prefix[b], wl.window_of(b), p))[0]
        k, v = full(pos)
        key = pos.tobytes()

        def hist(req):
            req = np.asarray(req, dtype=np.int64)
            assert req.tobytes() == key
            return k, v
        return hist

    done, elapsed = 0, 0.0
    with threadpool_limits(limits=1):
        while done < wl.batch and (elapsed < budget_s or done == 0):
            b = done
            h = prepared(b)
            t0 = time.perf_counter()
            attn.decode_query(q_rows[b], n_now[b] - 1, h, wl.prefix[b], wl.window_of(b),
                              wl.n_kv_heads, wl.rope_base, wl.scale)
            elapsed += time.perf_counter() - t0
            done += 1
    return {"value": done / elapsed, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} of {wl.batch} sequences of one decode step (all {wl.n_q_heads} "
                      f"query heads, float64 NumPy, 1 thread), {elapsed:.1f} s"}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def bench_prefill(calls: int, warmup: int = 2):
    """Chunked prefill: 8 sequences each take a 512-token chunk at t ~ U{8192..65536}.

    Each call attends the chunk (staging, MFMA attention) and appends it; the state
    advances by 512 tokens per call. Algorithmic work per call: 4 * H_q * D * sum over
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(run one process per GPU; sequences and KV heads shard with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import prefix_pinned_sliding_amd as psa
    from synth import configs, drive, gen

    torch.cuda.set_device(0)
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
    print(f"[bench] {wl.name}: filling {sum(n0)} tokens", file=sys.stderr, flush=True)
    if args.workload == "decode_shared_p2000":
        c = drive.make_cache(wl, n_shared=1, shared_max=wl.prefix[0], prefix_max=0, pe=args.pe)
    else:
        c = drive.make_cache(wl, pe=args.pe)
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

    def step(i):
        c.append(ks[i], vs[i])
        c.decode(qs[i], out)

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
    n_prof = [n + total for n in n0]          # history length during the last profiled step
    elem = 2 if wl.dtype == torch.bfloat16 else 4
    vis_first = wl.visible_tokens([n + args.warmup + args.steps + 1 for n in n0])
    vis_last = wl.visible_tokens(n_prof)
    vis = 0.5 * (vis_first + vis_last)
    launch_bytes = vis * wl.n_kv_heads * wl.head_dim * 2 * elem
    achieved = launch_bytes / dec_avg_s / 1e9
    traffic = load_traffic(launch_bytes)

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
                   "position_encoding": args.pe},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "kernel": "decode_partial",
                     "kernel_avg_us": dec_avg_s * 1e6, "bytes_per_launch": launch_bytes},
        "kernels_avg_us": {k: (ms / n * 1e3 if n else None) for k, (ms, n) in times.items()},
    }

    if not args.no_prefill and args.workload == "decode_p100_w4096":
        del c
        torch.cuda.empty_cache()
        print("[bench] chunked prefill", file=sys.stderr, flush=True)
        result["prefill"] = bench_prefill(args.prefill_calls)

    if not args.no_train and args.workload == "decode_p100_w4096":
        torch.cuda.empty_cache()
        print("[bench] training attention", file=sys.stderr, flush=True)
        result["train"] = bench_train(args.train_calls)

    if not args.no_cpu_baseline:
        qc = qs[total - 1].double().cpu().numpy()
        result["cpu_baseline"] = cpu_baseline(wl, n_prof, qc, args.cpu_seconds)

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
