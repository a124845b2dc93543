#!/usr/bin/env python3
"""Benchmark of the FP4 KV-cache decode path on one MI355X.

Default workload: 32 sequences of 32768 tokens, 64 query heads over 8 KV heads
(group 8), head dim 128, 64 context splits -- 1.2 GB of packed cache, larger
than the GPU's last-level cache, so every step streams it from HBM.  A step
is one fp4kv_decode_attention call (split kernel + combine kernel; the split
kernel alone when there is one partial per row); for the paged workload it is
one fp4kv_decode_append_attention call, whose split kernel first stores each
sequence's new token (--unfused: a separate quantize_append call, then
decode_attention).  The per-kernel breakdown runs the same steps as their
halves with events between launches.  The cache, the queries and every
argument are resident on the device before timing starts.

Prints one JSON line: achieved HBM GB/s over the step's algorithmic bytes
(packed K/V read, queries read, outputs written, page-table and length
entries read), decode steps/s, the split kernel's roofline figures, and the
CPU oracle's rate on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--splits S]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4-KV decode attention: achieved HBM GB/s (% of peak) and decode steps/s"
PEAK_HBM_GBS = 8000.0                       # MI355X HBM3E peak, GB/s
SETTLE_CALLS = 100                          # untimed decode calls before the warm-up steps
# sources of the split kernel (per cache format) whose HBM counters profiles/ may hold
_CSRC = os.path.join(ROOT, "fp4_quantised_kv_amd", "csrc")
KERNEL_SOURCES = {
    "fp4": ["fp4kv_decode_mfma.hip", "fp4kv_mfma_util.h", "fp4kv_merge.h", "fp4kv_internal.h", "fp4kv_quant.h"],
    "fp8": ["fp4kv_decode_fp8.hip", "fp4kv_mfma_util.h", "fp4kv_merge.h", "fp4kv_internal.h", "fp4kv_quant.h"],
}
KERNEL_SOURCES["fp8t"] = KERNEL_SOURCES["fp8"]
FORMAT_NAMES = {"fp4": "fp4_e2m1_e4m3_per16", "fp8": "fp8_e4m3_per_tensor_scale",
                "fp8t": "fp8_e4m3_per_token_fp16_scale"}
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_digest(fmt: str = "fp4") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[fmt]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counter_file(workload: str, fmt: str) -> str:
    prefix = {"fp4": "decode_split", "fp8": "decode_split_fp8", "fp8t": "decode_split_fp8_token"}[fmt]
    return os.path.join(PROFILES, f"{prefix}_{workload}_hbm_counters.txt")


def measured_traffic(workload: str, fmt: str = "fp4"):
    """Per-launch HBM bytes of the split kernel from the committed counter
    summary, if it was taken from the current kernel source; else None."""
    path = _counter_file(workload, fmt)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_source_sha256_16") != kernel_source_digest(fmt):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, seed, threads, fmt="fp4"):
    """The oracle (fp64 decode attention from its own codes) on a bounded
    sample: whole sequences of the workload, all their KV heads."""
    import numpy as np
    import fp4kv_workloads as wl
    import oracle
    lens = wl.seq_lengths(w, seed)
    # every sequence (about 10-15 s of oracle time at the 32K batch); the
    # per-token FP8 oracle holds float64 values, so a quarter of them there
    n_seq = w.batch if fmt != "fp8t" else min(w.batch, max(1, threads // 2))
    seqs = list(range(n_seq))
    q = wl.queries(w, seed)
    kc, ks, vc, vs = [], [], [], []
    budget_tokens = 1 << 17                    # cap the sample at 131072 tokens per sequence
    sample_lens = [min(int(lens[b]), budget_tokens) for b in range(w.batch)]
    k_scale, v_scale = wl.fp8_tensor_scales(w, seed)
    for b in range(w.batch):
        if b in seqs:
            k = wl.kv_tokens(w, seed, b, "k", 0, sample_lens[b])
            v = wl.kv_tokens(w, seed, b, "v", 0, sample_lens[b])
            if fmt == "fp8t":
                (a, sa), (c, sc) = (oracle.quantize_fp8_groups(wl.bf16_bits(k), "token"),
                                    oracle.quantize_fp8_groups(wl.bf16_bits(v), "token"))
            elif fmt == "fp8":
                a, c = oracle.quantize_fp8(wl.bf16_bits(k), k_scale), oracle.quantize_fp8(wl.bf16_bits(v), v_scale)
                sa = sc = None
            else:
                a, sa, _ = oracle.quantize(wl.bf16_bits(k), want_xhat=False, n_threads=threads)
                c, sc, _ = oracle.quantize(wl.bf16_bits(v), want_xhat=False, n_threads=threads)
        else:
            a = c = np.zeros((0, w.kv_heads, w.head_dim), np.uint8)
            sa = sc = np.zeros((0, w.kv_heads, w.head_dim // 16), np.uint8)
        kc.append(a); ks.append(sa); vc.append(c); vs.append(sc)
    heads = [(b, h) for b in seqs for h in range(w.kv_heads)]
    t0 = time.perf_counter()
    if fmt == "fp8t":
        # the stored values (E4M3 codes times each token's fp16 scale), then attention
        deq = lambda x, s_: (oracle.dequantize_fp8_groups(x, s_, "token") if x.shape[0]
                             else np.zeros((1, w.kv_heads, w.head_dim)))
        kv = [deq(x, s_) for x, s_ in zip(kc, ks)]
        vv = [deq(x, s_) for x, s_ in zip(vc, vs)]
        oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, sample_lens, w.head_dim ** -0.5,
                                       heads=heads, n_threads=threads)
    elif fmt == "fp8":
        oracle.decode_attention_fp8(wl.bf16_bits(q), kc, vc, k_scale, v_scale, sample_lens, w.head_dim ** -0.5,
                                    heads=heads, n_threads=threads)
    else:
        oracle.decode_attention(wl.bf16_bits(q), kc, ks, vc, vs, sample_lens, w.head_dim ** -0.5,
                                heads=heads, n_threads=threads)
    dt = time.perf_counter() - t0
    tokens = sum(sample_lens[b] for b in seqs)
    per_number = {"fp4": 9 / 16, "fp8": 1.0, "fp8t": 1.0 + 2.0 / w.head_dim}[fmt]
    bytes_ = int(tokens * 2 * w.kv_heads * w.head_dim * per_number) + n_seq * w.q_heads * w.head_dim * 6
    return {"value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_seq} of {w.batch} sequences, {tokens} tokens, all {w.kv_heads} KV heads; "
                      f"decode attention from the oracle's own codes in fp64, {dt:.2f} s wall"}


def prefill_append(fk, wl, seed, dev, stream, reps=10):
    """quantize_append of the prefill workload (8 sequences x 8192 tokens,
    H_kv 8, D 128, contiguous slots) as one call; bf16 K, V read + packed
    bytes written, per call."""
    import torch
    w = wl.WORKLOADS["prefill_b8_8k"]
    fkk, fvv = wl.channel_factors(w, seed, "k"), wl.channel_factors(w, seed, "v")
    k = torch.cat([wl.kv_tokens(w, seed, b, "k", 0, w.context, fkk) for b in range(w.batch)]).to(dev)
    v = torch.cat([wl.kv_tokens(w, seed, b, "v", 0, w.context, fvv) for b in range(w.batch)]).to(dev)
    n = k.shape[0]
    layout = fk.cache_layout(w.kv_heads, w.head_dim, -(-n // 64))
    cache = torch.empty(layout.cache_bytes, dtype=torch.uint8, device=dev)
    slots = torch.arange(n, dtype=torch.int64, device=dev)
    fk.quantize_append(layout, k, v, slots, cache)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fk.quantize_append(layout, k, v, slots, cache)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    bytes_ = 2 * k.numel() * 2 + layout.cache_bytes + n * 8
    return {"workload": w.name, "tokens": n, "ms": round(ms, 5), "gbs": round(bytes_ / (ms * 1e-3) / 1e9, 1),
            "algorithmic_bytes": bytes_}


def cold_and_warm(fk, gc, w, seed, dev, stream, splits_req, step_bytes, reps=20):
    """For a cache smaller than the 256 MB last-level cache: decode step
    (one fp4kv_decode_attention call) time warm (back to back: the cache stays in the
    last-level cache) and cold (1 GiB of unrelated data read and written
    between calls, outside the timed events, so every call reads the cache
    from HBM).  Steps this small take less GPU time than the host needs to
    enqueue them, so both measurements queue their calls behind GPU work
    that is still running (a spin kernel that touches no memory, or the
    scrub) and time the GPU, not the host."""
    import torch
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    splits, partials, ws_bytes = fk.decode_plan(gc.layout, B, Hq, gc.page_table.shape[1], splits_req)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    import fp4kv_workloads as wl
    q = wl.queries(w, seed).to(dev)
    scrub = torch.zeros(1 << 28, dtype=torch.int32, device=dev)     # 1 GiB

    def call():
        fk.decode_attention(gc.layout, gc.cache, q, gc.seq_lens, gc.page_table, num_splits=splits_req,
                            workspace=ws, out=out)

    for _ in range(5):
        call()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)                  # ~1 ms of GPU clock cycles while the calls are enqueued
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) / reps
    cold = []
    for _ in range(reps):
        scrub.add_(1)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        call()
        c1.record(stream)
        torch.cuda.synchronize()
        cold.append(c0.elapsed_time(c1))
    cold_ms = sorted(cold)[len(cold) // 2]
    del scrub
    return {"cache_bytes": gc.layout.cache_bytes, "step_bytes": int(step_bytes),
            "warm_ms": round(warm, 5), "warm_gbs": round(step_bytes / (warm * 1e-3) / 1e9, 1),
            "cold_ms_median": round(cold_ms, 5), "cold_ms_min": round(min(cold), 5),
            "cold_gbs": round(step_bytes / (cold_ms * 1e-3) / 1e9, 1),
            "note": "warm: back-to-back steps; cold: 1 GiB scrubbed through the caches before each step"}


def copy_ceiling(dev, stream, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy (read + write) of nbytes: the rate a
    kernel that reads and writes HBM in equal measure can expect."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    return {"bytes_read_and_written": 2 * nbytes, "ms": round(ms, 5), "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def query_extras(fk, gc, w, dev, stream, splits_req, reps=20, window=4096):
    """On the workload's cache: causal attention of S = 16 / G query tokens
    per sequence in one pass (speculative verification), and sliding-window
    attention over the last `window` tokens.  Rates over the bytes each call
    must move (cache pages read, queries, outputs)."""
    import torch
    L, B, Hq, D = gc.layout, w.batch, w.q_heads, w.head_dim
    S = max(1, 16 // w.group)
    g = torch.Generator(device=dev).manual_seed(7)
    q = torch.randn(B, S, Hq, D, generator=g, device=dev).to(torch.bfloat16)
    lens = [int(x) for x in gc.lens_cpu]
    out = {}
    for name, win in (("multi_query", 0), ("window", window)):
        plan = fk.decode_window_plan(L, B, S if name == "multi_query" else 1, Hq, gc.page_table.shape[1], win,
                                     splits_req if win == 0 else 0)
        ws = torch.empty(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
        qq = q if name == "multi_query" else q[:, :1].contiguous()
        S_ = qq.shape[1]
        res = torch.empty(B, S_, Hq, D, dtype=torch.float32, device=dev)
        call = lambda: fk.decode_window_attention(L, gc.cache, qq, gc.seq_lens, gc.page_table, win,
                                                  num_splits=splits_req if win == 0 else 0, workspace=ws, out=res)
        for _ in range(3):
            call()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tokens = [min(n, win + S_ - 1) if win else n for n in lens]
        bytes_ = sum(tokens) * L.bytes_per_token + B * S_ * Hq * D * (2 + 4) + sum(-(-t // 64) for t in tokens) * 4
        out[name] = {"q_tokens": S_, "window": win, "ms": round(ms, 5), "gbs": round(bytes_ / (ms * 1e-3) / 1e9, 1),
                     "query_tokens_per_s": round(B * S_ / (ms * 1e-3), 1), "algorithmic_bytes": int(bytes_)}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gqa8_b32_ctx32k")
    ap.add_argument("--splits", type=int, default=None, help="context splits (default: the workload's)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--format", choices=("fp4", "fp8", "fp8t"), default="fp4",
                    help="cache format: FP4 E2M1 + E4M3 per 16 (default), FP8 E4M3 with per-tensor scales, "
                         "or FP8 E4M3 with an fp16 scale per token (fp8t)")
    ap.add_argument("--unfused", action="store_true",
                    help="paged workload: append with quantize_append, then decode (default: the decode "
                         "kernel stores the new tokens itself)")
    ap.add_argument("--kernel", choices=("auto", "mfma_staged", "mfma_direct", "valu"),
                    default="auto", help="split kernel of the timed steps (through fp4kv_decode_with_options "
                                         "unless auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the streaming-read probe (the achievable HBM read rate for this access pattern)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill quantise-append measurement (8 x 8192 tokens)")
    ap.add_argument("--extras", action="store_true",
                    help="also time several query tokens in one pass and sliding-window attention on the cache")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="finish with one 1 GiB device copy, the known-size kernel for scaling HBM counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode path shards by sequence and KV head with no "
              "exchange, so a multi-GPU figure is N independent copies of this one; run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import fp4_quantised_kv_amd as fk
    import fp4kv_harness as hx
    import fp4kv_workloads as wl

    if not os.path.exists(fk.LIBRARY_PATH):
        from fp4_quantised_kv_amd import build as hip_build
        hip_build.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    w = wl.WORKLOADS[args.workload]
    if w.kind == "prefill":
        raise SystemExit("the prefill workload is timed by its own test, not as a decode step")
    splits_req = w.splits if args.splits is None else args.splits
    paged = w.kind == "paged"
    total_steps = args.warmup + args.steps
    t_setup = time.perf_counter()
    print(f"# building cache for {w.name}: {w.description}", file=sys.stderr, flush=True)
    gc = hx.build_cache(w, args.seed, extra_tokens=total_steps if paged else 0, zero=False, fmt=args.format)
    print(f"# cache built in {time.perf_counter() - t_setup:.1f} s "
          f"({gc.layout.cache_bytes / 1e9:.3f} GB)", file=sys.stderr, flush=True)
    L = gc.layout
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    max_pages = gc.page_table.shape[1]
    splits, partials, ws_bytes = fk.decode_plan(L, B, Hq, max_pages, splits_req)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
    lens0 = gc.lens_cpu.clone()

    # per-step inputs, all on the device before timing
    qs = [wl.queries(w, args.seed, step=s if paged else 0).to(dev) for s in range(total_steps if paged else 1)]
    if paged:
        news, slots, lens_dev = [], [], []
        for s in range(total_steps):
            kn, vn = wl.new_tokens(w, args.seed, s)
            sl = torch.stack([wl.slots_for(gc.pt_cpu.table, b, int(lens0[b]) + s, int(lens0[b]) + s + 1)[0]
                              for b in range(B)])
            news.append((kn.to(dev), vn.to(dev)))
            slots.append(sl.to(dev))
            lens_dev.append((lens0 + s + 1).to(torch.int32).to(dev))
    else:
        lens_dev = [gc.seq_lens]
    scale = D ** -0.5
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(total_steps)]

    fused = paged and not args.unfused

    def step_call(s):
        # one step through the library's entry point, as a caller makes it
        if args.kernel != "auto":
            if paged and not fused:
                fk.quantize_append(L, news[s][0], news[s][1], slots[s], gc.cache)
            kv = dict(k_new=news[s][0], v_new=news[s][1]) if paged and fused else {}
            fk.decode_with_options(L, gc.cache, qs[s % len(qs)], lens_dev[s % len(lens_dev)], gc.page_table,
                                   softmax_scale=scale, num_splits=splits_req, workspace=ws, out=out,
                                   kernel=args.kernel, **kv)
            return
        if paged and fused:
            fk.decode_append_attention(L, gc.cache, news[s][0], news[s][1], qs[s % len(qs)], lens_dev[s],
                                       gc.page_table, softmax_scale=scale, num_splits=splits_req, workspace=ws,
                                       out=out)
            return
        if paged:
            fk.quantize_append(L, news[s][0], news[s][1], slots[s], gc.cache)
        fk.decode_attention(L, gc.cache, qs[s % len(qs)], lens_dev[s % len(lens_dev)], gc.page_table,
                            softmax_scale=scale, num_splits=splits_req, workspace=ws, out=out)

    def step(s, e=None):
        """The same step as its halves (split kernel, then combine), with
        events between the launches for the per-kernel breakdown."""
        if e is not None:
            e[0].record(stream)
        if paged and not fused:
            fk.quantize_append(L, news[s][0], news[s][1], slots[s], gc.cache)
        if e is not None:
            e[1].record(stream)
        if fused:
            # the split kernel stores each sequence's new token itself
            fk.decode_append_split(L, gc.cache, news[s][0], news[s][1], qs[s % len(qs)], lens_dev[s],
                                   gc.page_table, softmax_scale=scale, num_splits=splits_req, workspace=ws)
        else:
            fk.decode_split(L, gc.cache, qs[s % len(qs)], lens_dev[s % len(lens_dev)], gc.page_table,
                            softmax_scale=scale, num_splits=splits_req, workspace=ws)
        if e is not None:
            e[2].record(stream)
        fk.decode_combine(ws, B, Hq, D, partials, out=out)
        if e is not None:
            e[3].record(stream)

    # Clock settle, before the warm-up steps: the GPU reaches its steady
    # clocks only after tens of milliseconds of load (100 decode calls take
    # ~20 ms here; with 5 warm-up steps alone the first timed steps run ~8 %
    # slower).  Decode only, so the paged cache is not changed.
    for _ in range(SETTLE_CALLS):
        fk.decode_split(L, gc.cache, qs[0], gc.seq_lens, gc.page_table, softmax_scale=scale,
                        num_splits=splits_req, workspace=ws)
        fk.decode_combine(ws, B, Hq, D, partials, out=out)
    torch.cuda.synchronize()
    for s in range(args.warmup):
        step_call(s)
    torch.cuda.synchronize()
    # the timed region: K steps with no event between their launches
    t0 = time.perf_counter()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for s in range(args.warmup, total_steps):
        step_call(s)
    stop.record(stream)
    host_enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / args.steps

    # per-kernel breakdown: the same steps again (appends rewrite the same
    # slots with the same bytes), with an event between launches
    for s in range(args.warmup, total_steps):
        step(s, ev[s])
    torch.cuda.synchronize()
    timed = ev[args.warmup:]
    t_append = sum(e[0].elapsed_time(e[1]) for e in timed) / args.steps
    t_split = sum(e[1].elapsed_time(e[2]) for e in timed) / args.steps
    t_comb = sum(e[2].elapsed_time(e[3]) for e in timed) / args.steps

    # the split kernel alone, launched back to back with no event between
    # launches: its average duration for the roofline figure
    last = total_steps - 1
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        fk.decode_split(L, gc.cache, qs[last % len(qs)], lens_dev[last % len(lens_dev)], gc.page_table,
                        softmax_scale=scale, num_splits=splits_req, workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    t_split_b2b = e0.elapsed_time(e1) / args.steps

    # algorithmic bytes
    if paged:
        ctx = [int(lens0[b]) + args.warmup + 1 for b in range(B)]   # mid-run lengths, +1 per step
        ctx_tokens = sum(ctx) + B * (args.steps - 1) / 2.0
    else:
        ctx = [int(x) for x in lens0]
        ctx_tokens = float(sum(ctx))
    pages_read = sum(-(-c // 64) for c in ctx)
    cache_read = ctx_tokens * L.bytes_per_token
    split_bytes = cache_read + B * Hq * D * 2 + pages_read * 4 + B * 4
    step_bytes = split_bytes + B * Hq * D * 4
    if paged:
        step_bytes += B * w.kv_heads * D * 2 * 2 + B * L.bytes_per_token + B * 8
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    # the back-to-back launches all attend over the last step's lengths
    if paged:
        ctx_last = [int(lens0[b]) + total_steps for b in range(B)]
        split_bytes_b2b = (sum(ctx_last) * L.bytes_per_token + B * Hq * D * 2
                           + sum(-(-c // 64) for c in ctx_last) * 4 + B * 4)
    else:
        split_bytes_b2b = split_bytes
    split_gbs = split_bytes_b2b / (t_split_b2b * 1e-3) / 1e9
    traffic = measured_traffic(w.name, args.format)

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": w.kv_heads,
                   "head_dim": D, "context": w.context if not paged else f"{w.min_len}..{w.max_len}",
                   "format": FORMAT_NAMES[args.format],
                   "splits": splits, "partials": partials, "page_size": 64,
                   "cache_bytes": L.cache_bytes},
        "decode_steps_per_s": round(1e3 / ms_per_step, 2),
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "append": (None if not paged else "fused into the split kernel" if fused else "quantize_append"),
        "kernel": args.kernel,
        "kernel_ms": {"append": round(t_append, 5), "decode_split": round(t_split, 5),
                      "decode_combine": round(t_comb, 5), "decode_split_back_to_back": round(t_split_b2b, 5)},
        "settle_decode_calls": SETTLE_CALLS,
        "wall_s_timed": round(wall, 4),
        "host_enqueue_ms_per_step": round(1e3 * host_enqueue / args.steps, 5),
        "roofline": {"bound": "hbm",
                     "kernel": ("decode_split_fp8" if args.format == "fp8" else
                                "decode_split_fp8 (per-token scales)" if args.format == "fp8t" else
                                "decode_split_mfma<128, staged>" if D == 128 else "decode_split_mfma<64>"),
                     "achieved": round(split_gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(split_gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": int(split_bytes_b2b)},
    }
    if not args.no_prefill:
        result["prefill_append"] = prefill_append(fk, wl, args.seed, dev, stream)
        result["prefill_append"]["device_copy"] = copy_ceiling(dev, stream)
    if L.cache_bytes < (256 << 20) and not paged:
        result["cold_warm"] = cold_and_warm(fk, gc, w, args.seed, dev, stream, splits_req, step_bytes)
    if args.extras and not paged:
        result["extras"] = query_extras(fk, gc, w, dev, stream, splits_req)
    if not args.no_read_probe:
        # the achievable read rate: the cache's size in 9216-byte blocks,
        # streamed once by the library's read probe
        buf = torch.full((L.cache_bytes // 9216 * 9216,), 1, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        for _ in range(3):
            fk.read_probe(buf, sink)
        e0.record(stream)
        for _ in range(10):
            fk.read_probe(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        result["hbm_read_probe"] = {"kernel": "read_probe: 16-byte loads, one 9216-byte block per wave",
                                    "bytes": buf.numel(),
                                    "gbs": round(buf.numel() * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)}
        result["roofline"]["frac_of_read_probe"] = round(split_gbs / result["hbm_read_probe"]["gbs"], 4)
        del buf
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = src.numel()
        del src, dst
    if not args.no_cpu_baseline:
        threads = max(1, min(16, os.cpu_count() or 1))
        result["cpu_baseline"] = cpu_baseline(w, args.seed, threads, args.format)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
