#!/usr/bin/env python3
"""Benchmark of the FP4 KV-cache decode path on one MI355X.

Headline workload: 32 sequences of 32768 tokens, 64 query heads over 8 KV
heads (group 8), head dim 128, 64 context splits -- 1.2 GB of packed cache,
larger than the GPU's last-level cache, so every step streams it from HBM.  A
step is one decode-attention call (split kernel + combine kernel; the split
kernel alone when there is one partial per row) through
fp4kv_decode_with_options, given the batch's shortest length (min_seq_len:
host knowledge a serving caller has; it only sizes the context chunks, and
sends a uniform batch's last workgroups one-page chunks).  For the paged
workload the call appends: its split kernel first stores each sequence's new
token (--unfused: a separate quantize_append call, then the decode).  The
same step through the plain entry point (fp4kv_decode_attention or
fp4kv_decode_append_attention, which know no lengths) is timed beside it and
reported as "plain_entry_point"; --no-length-hint times the plain calls'
chunking throughout.  The per-kernel breakdown runs the same steps as their
halves with events between launches.  The cache, the queries and every
argument are resident on the device before timing starts.

Prints one JSON line: achieved HBM GB/s over the step's algorithmic bytes
(packed K/V read, queries read, outputs written, page-table and length
entries read), decode steps/s, the split kernel's roofline figures, the
achievable read rate (a sweep of streaming-read probes), the CPU oracle's
rate on a bounded sample of the same workload, and under "configs" the same
figures for the other workloads: the 256-token and 4096-token batches (cold
and warm: their caches fit the last-level cache), the 512K-token sequence,
the paged batch and the prefill quantise-append.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--splits S]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4-KV decode attention: achieved HBM GB/s (% of peak) and decode steps/s"
PEAK_HBM_GBS = 8000.0                       # MI355X HBM3E peak, GB/s
SETTLE_CALLS = 100                          # untimed decode calls before the warm-up steps
# The arithmetic of the decode path: dequantised K and V (exact in fp16) and
# the query (times a power of two, exact) as fp16 matrix-core operands,
# probabilities as two fp16 parts, fp32 accumulation and softmax.
DTYPE = "f16 MFMA operands, f32 accumulate"
LLC_BYTES = 256 << 20                       # MI355X last-level (Infinity) cache
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
# the other workloads reported under "configs"
SUB_CONFIGS = ("tiny_d64_ctx256", "gqa4_b8_ctx4k", "gqa4_b1_ctx512k", "paged_b64_len1k_16k")


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


def oracle_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, capped by the
    per-GPU CPU share the environment states in OMP_NUM_THREADS, if set."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        share = 0
    return max(1, min(avail, share) if share > 0 else avail)


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
    host = os.cpu_count()
    return {"value": round(bytes_ / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "threads": threads,
            "host_cpus": host, "kind": "oracle",
            "sample": f"{n_seq} of {w.batch} sequences, {tokens} tokens, all {w.kv_heads} KV heads; "
                      f"decode attention from the oracle's own codes in fp64 on {threads} threads "
                      f"(the CPUs given to this process; the host shows {host}), {dt:.2f} s wall"}


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _time(torch, stream, call, reps, warm=3):
    """Average ms of `reps` back-to-back calls after `warm` untimed ones."""
    for _ in range(warm):
        call()
    e0, e1 = _events(torch)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def prefill_append(fk, wl, seed, dev, stream, reps=10):
    """quantize_append of the prefill workload (8 sequences x 8192 tokens,
    H_kv 8, D 128, contiguous slots) as one call; bf16 K, V read + packed
    bytes written + slots read, per call.  The kernel reads and writes HBM,
    so its ceiling is a device copy, timed beside it."""
    import torch
    w = wl.WORKLOADS["prefill_b8_8k"]
    fkk, fvv = wl.channel_factors(w, seed, "k"), wl.channel_factors(w, seed, "v")
    k = torch.cat([wl.kv_tokens(w, seed, b, "k", 0, w.context, fkk) for b in range(w.batch)]).to(dev)
    v = torch.cat([wl.kv_tokens(w, seed, b, "v", 0, w.context, fvv) for b in range(w.batch)]).to(dev)
    n = k.shape[0]
    layout = fk.cache_layout(w.kv_heads, w.head_dim, -(-n // 64))
    cache = torch.empty(layout.cache_bytes, dtype=torch.uint8, device=dev)
    slots = torch.arange(n, dtype=torch.int64, device=dev)
    ms = _time(torch, stream, lambda: fk.quantize_append(layout, k, v, slots, cache), reps)
    bytes_ = 2 * k.numel() * 2 + layout.cache_bytes + n * 8
    gbs = bytes_ / (ms * 1e-3) / 1e9
    del k, v, cache
    copy = copy_ceiling(dev, stream)
    ceil = stream_ceiling(fk, dev, stream, 2 * n * w.kv_heads * w.head_dim * 2, layout.cache_bytes)
    return {"workload": w.name, "tokens": n, "ms": round(ms, 5), "gbs": round(gbs, 1),
            "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2), "algorithmic_bytes": bytes_,
            "roofline": {"bound": "hbm", "kernel": "append_slices_kernel<128>", "achieved": round(gbs, 2),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": prefill_traffic(), "algorithmic_bytes_per_launch": bytes_,
                         "frac_of_stream_ceiling": round(gbs / ceil["coalesced"]["gbs"], 4),
                         "frac_of_paired_load_ceiling": round(gbs / ceil["paired"]["gbs"], 4)},
            "stream_ceiling": ceil, "device_copy": copy}


def stream_ceiling(fk, dev, stream, read_total, write_total, reps=10):
    """The achievable rate of the prefill's traffic: streaming probes that
    read and write in its proportion, one wave per 16-token slice's worth
    (64 KB of bf16 K and V in, a quarter of that plus the scales out), with
    whole-kilobyte loads (coalesced) and with the quantiser's own pattern (a
    16-channel block's 32 bytes per lane as two 16-byte loads: paired); the
    fastest grid of each."""
    import torch
    unit_r = 65536
    units = read_total // unit_r
    unit_w = -(-write_total // units // 1024) * 1024
    src = torch.full((units * unit_r,), 1, dtype=torch.uint8, device=dev)
    dst = torch.empty(units * unit_w, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for name, paired in (("coalesced", False), ("paired", True)):
        best = None
        for groups in (1024, 2048, 4096):
            ms = _time(torch, stream, lambda: fk.stream_probe(src, dst, unit_r, unit_w, paired, groups, sink), reps)
            g = units * (unit_r + unit_w) / (ms * 1e-3) / 1e9
            if best is None or g > best["gbs"]:
                best = {"gbs": round(g, 1), "ms": round(ms, 5), "workgroups": groups}
        out[name] = best
    out["per_wave_unit"] = {"read_bytes": unit_r, "write_bytes": unit_w, "units": units}
    del src, dst
    return out


def prefill_traffic():
    """Per-launch HBM bytes of the prefill quantiser from the committed
    counter summary, if taken from the current source; else None."""
    path = os.path.join(PROFILES, "append_prefill_b8_8k_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            fields[key.strip()] = val.strip()
    if fields.get("kernel_source_sha256_16") != quantiser_source_digest():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def quantiser_source_digest() -> str:
    h = hashlib.sha256()
    for name in ("fp4kv_kernels.hip", "fp4kv_quant.h", "fp4kv_internal.h"):
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def copy_ceiling(dev, stream, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy (read + write) of nbytes: the rate a
    kernel that reads and writes HBM in equal measure can expect."""
    import torch
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    ms = _time(torch, stream, lambda: dst.copy_(src), reps)
    return {"bytes_read_and_written": 2 * nbytes, "ms": round(ms, 5), "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def read_ceiling(fk, dev, stream, nbytes, reps=10):
    """The achievable HBM read rate: streaming-read probes over a buffer of
    about nbytes (larger than the last-level cache, read once per call),
    swept over loads in flight per lane, workgroups and destination
    (registers, or LDS as the decode kernels copy pages); the fastest is the
    ceiling.  Also the library's fixed-shape read probe."""
    import torch
    nbytes = max(nbytes, 2 * LLC_BYTES) // 16384 * 16384
    buf = torch.full((nbytes,), 1, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    sweep = []
    for to_lds in (False, True):
        for loads in ((4, 8, 16) if not to_lds else (4, 8)):
            for groups in (512, 1024, 2048, 4096):
                ms = _time(torch, stream, lambda: fk.read_probe_config(buf, sink, loads, groups, to_lds), reps)
                sweep.append({"dest": "lds" if to_lds else "regs", "loads_per_lane": loads, "workgroups": groups,
                              "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)})
    fixed = buf[: nbytes // 9216 * 9216]
    ms = _time(torch, stream, lambda: fk.read_probe(fixed, sink), reps)
    fixed_gbs = round(fixed.numel() / (ms * 1e-3) / 1e9, 1)
    best = max(sweep, key=lambda r: r["gbs"])
    del buf, fixed
    return {"kernel": "read_probe_regs / read_probe_lds: 16-byte non-temporal loads, one pass, grid-stride",
            "bytes": nbytes, "gbs": best["gbs"], "pct_of_peak_hbm": round(100.0 * best["gbs"] / PEAK_HBM_GBS, 2),
            "best": best, "fixed_shape_read_probe_gbs": fixed_gbs, "sweep": sweep}


class DecodeRun:
    """One decode workload's cache on the device, its per-step inputs and the
    calls that make a step."""

    def __init__(self, fk, hx, wl, w, seed, fmt, dev, n_steps, splits=None, unfused=False, kernel="auto",
                 length_hint=True):
        import torch
        self.fk, self.w, self.fmt, self.dev = fk, w, fmt, dev
        self.paged = w.kind == "paged"
        self.fused = self.paged and not unfused
        self.kernel = kernel
        self.length_hint = length_hint
        self.splits_req = w.splits if splits is None else splits
        t_setup = time.perf_counter()
        print(f"# building cache for {w.name}: {w.description}", file=sys.stderr, flush=True)
        self.gc = gc = hx.build_cache(w, seed, extra_tokens=n_steps if self.paged else 0, zero=False, fmt=fmt)
        print(f"# cache built in {time.perf_counter() - t_setup:.1f} s "
              f"({gc.layout.cache_bytes / 1e9:.3f} GB)", file=sys.stderr, flush=True)
        L = gc.layout
        B, Hq, D = w.batch, w.q_heads, w.head_dim
        self.splits, self.partials, ws_bytes = fk.decode_plan(L, B, Hq, gc.page_table.shape[1], self.splits_req)
        self.ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.out = torch.empty(B, Hq, D, dtype=torch.float32, device=dev)
        self.lens0 = gc.lens_cpu.clone()
        # the shortest length of every step (a paged step adds one token per sequence first)
        self.min_len = int(self.lens0.min()) + (1 if self.paged else 0) if length_hint else 0
        self.scale = D ** -0.5
        # per-step inputs, all on the device before timing
        self.qs = [wl.queries(w, seed, step=s if self.paged else 0).to(dev) for s in range(n_steps if self.paged else 1)]
        if self.paged:
            self.news, self.slots, self.lens_dev = [], [], []
            for s in range(n_steps):
                kn, vn = wl.new_tokens(w, seed, s)
                sl = torch.stack([wl.slots_for(gc.pt_cpu.table, b, int(self.lens0[b]) + s,
                                               int(self.lens0[b]) + s + 1)[0] for b in range(B)])
                self.news.append((kn.to(dev), vn.to(dev)))
                self.slots.append(sl.to(dev))
                self.lens_dev.append((self.lens0 + s + 1).to(torch.int32).to(dev))
        else:
            self.lens_dev = [gc.seq_lens]

    def q(self, s):
        return self.qs[s % len(self.qs)]

    def lens(self, s):
        return self.lens_dev[s % len(self.lens_dev)]

    def chunks(self):
        """The chunk cut the steps use (fp4kv_decode_chunks)."""
        w = self.w
        return self.fk.decode_chunks(self.gc.layout, w.batch, w.q_heads, self.gc.page_table.shape[1],
                                     self.splits_req, min_seq_len=self.min_len)

    def step(self, s):
        """One step through the library's entry point, as a caller makes it:
        with the batch's shortest length (and the kernel asked for)."""
        fk, gc, L = self.fk, self.gc, self.gc.layout
        if self.paged and not self.fused:
            fk.quantize_append(L, self.news[s][0], self.news[s][1], self.slots[s], gc.cache)
        kv = dict(k_new=self.news[s][0], v_new=self.news[s][1]) if self.fused else {}
        fk.decode_with_options(L, gc.cache, self.q(s), self.lens(s), gc.page_table, softmax_scale=self.scale,
                               num_splits=self.splits_req, workspace=self.ws, out=self.out, kernel=self.kernel,
                               min_seq_len=self.min_len, **kv)

    def plain_call(self):
        if self.kernel != "auto":
            return "fp4kv_decode_with_options (min_seq_len 0)"
        return "fp4kv_decode_append_attention" if self.fused else "fp4kv_decode_attention"

    def step_plain(self, s):
        """The same step through the entry point that knows no lengths (with
        an explicit kernel: the options call without a length)."""
        fk, gc, L = self.fk, self.gc, self.gc.layout
        if self.paged and not self.fused:
            fk.quantize_append(L, self.news[s][0], self.news[s][1], self.slots[s], gc.cache)
        if self.kernel != "auto":
            kv = dict(k_new=self.news[s][0], v_new=self.news[s][1]) if self.fused else {}
            fk.decode_with_options(L, gc.cache, self.q(s), self.lens(s), gc.page_table, softmax_scale=self.scale,
                                   num_splits=self.splits_req, workspace=self.ws, out=self.out, kernel=self.kernel,
                                   **kv)
        elif self.fused:
            fk.decode_append_attention(L, gc.cache, self.news[s][0], self.news[s][1], self.q(s), self.lens(s),
                                       gc.page_table, softmax_scale=self.scale, num_splits=self.splits_req,
                                       workspace=self.ws, out=self.out)
        else:
            fk.decode_attention(L, gc.cache, self.q(s), self.lens(s), gc.page_table, softmax_scale=self.scale,
                                num_splits=self.splits_req, workspace=self.ws, out=self.out)

    def append(self, s):
        if self.paged and not self.fused:
            self.fk.quantize_append(self.gc.layout, self.news[s][0], self.news[s][1], self.slots[s], self.gc.cache)

    def split(self, s, append=True):
        """The split kernel of step s as the step launches it (storing the
        step's new tokens itself when the step is fused and `append`)."""
        fk, gc, L = self.fk, self.gc, self.gc.layout
        kv = dict(k_new=self.news[s][0], v_new=self.news[s][1]) if self.fused and append else {}
        fk.decode_with_options(L, gc.cache, self.q(s), self.lens(s), gc.page_table, softmax_scale=self.scale,
                               num_splits=self.splits_req, workspace=self.ws, kernel=self.kernel, merge="none",
                               min_seq_len=self.min_len, **kv)

    def combine(self):
        w = self.w
        self.fk.decode_combine(self.ws, w.batch, w.q_heads, w.head_dim, self.partials, out=self.out)

    def split_bytes(self, ctx):
        """Algorithmic bytes of one split-kernel launch over context lengths
        `ctx`: packed K/V of every token, the queries, one page-table entry
        per page and one length per sequence."""
        L, w = self.gc.layout, self.w
        return (sum(ctx) * L.bytes_per_token + w.batch * w.q_heads * w.head_dim * 2
                + sum(-(-c // 64) for c in ctx) * 4 + w.batch * 4)

    def split_kernel_name(self):
        if self.fmt == "fp8":
            return "decode_split_fp8"
        if self.fmt == "fp8t":
            return "decode_split_fp8 (per-token scales)"
        return "decode_split_mfma<128, staged>" if self.w.head_dim == 128 else "decode_split_mfma<64>"


def decode_record(torch, run, stream, steps, warmup):
    """Time `steps` steps launched back to back (after a clock settle and
    `warmup` untimed steps), then the same steps as their halves with events
    between launches, then the split kernel alone back to back; returns the
    step's rate, the breakdown and the split kernel's roofline block.  For a
    cache larger than the last-level cache, so every step reads it from HBM."""
    w = run.w
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    # Clock settle, before the warm-up steps: the GPU reaches its steady
    # clocks only after tens of milliseconds of load (100 decode calls take
    # ~20 ms here; with 5 warm-up steps alone the first timed steps run ~8 %
    # slower).  Decode only, so the paged cache is not changed.
    for _ in range(SETTLE_CALLS):
        run.split(0, append=False)
        run.combine()
    torch.cuda.synchronize()
    for s in range(warmup):
        run.step(s)
    torch.cuda.synchronize()
    # the timed region: K steps with no event between their launches
    t0 = time.perf_counter()
    start, stop = _events(torch)
    start.record(stream)
    for s in range(warmup, warmup + steps):
        run.step(s)
    stop.record(stream)
    host_enqueue = time.perf_counter() - t0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / steps
    # the same steps through the plain entry point (no length known), back to
    # back; the paged appends rewrite the same slots with the same bytes
    e0, e1 = _events(torch)
    e0.record(stream)
    for s in range(warmup, warmup + steps):
        run.step_plain(s)
    e1.record(stream)
    torch.cuda.synchronize()
    t_plain = e0.elapsed_time(e1) / steps
    # per-kernel breakdown: the same steps again (appends rewrite the same
    # slots with the same bytes), with an event between launches
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i, s in enumerate(range(warmup, warmup + steps)):
        ev[i][0].record(stream)
        run.append(s)
        ev[i][1].record(stream)
        run.split(s)
        ev[i][2].record(stream)
        run.combine()
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    t_append = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    t_split = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    t_comb = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    # the split kernel alone, launched back to back with no event between
    # launches (over the last step's lengths): its average duration for the
    # roofline figure
    last = warmup + steps - 1
    e0, e1 = _events(torch)
    e0.record(stream)
    for _ in range(steps):
        run.split(last, append=False)
    e1.record(stream)
    torch.cuda.synchronize()
    t_split_b2b = e0.elapsed_time(e1) / steps

    if run.paged:
        ctx = [int(run.lens0[b]) + warmup + 1 for b in range(B)]   # mid-run lengths, +1 per step
        step_split = run.split_bytes(ctx) + B * (steps - 1) / 2.0 * run.gc.layout.bytes_per_token
        ctx_last = [int(run.lens0[b]) + warmup + steps for b in range(B)]
    else:
        ctx = ctx_last = [int(x) for x in run.lens0]
        step_split = run.split_bytes(ctx)
    step_bytes = step_split + B * Hq * D * 4
    if run.paged:
        step_bytes += B * w.kv_heads * D * 2 * 2 + B * run.gc.layout.bytes_per_token + B * 8
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    split_bytes_b2b = run.split_bytes(ctx_last)
    split_gbs = split_bytes_b2b / (t_split_b2b * 1e-3) / 1e9
    plain_gbs = step_bytes / (t_plain * 1e-3) / 1e9
    plain_call = run.plain_call()
    return {
        "workload": w.name, "ms_per_step": round(ms_per_step, 5), "gbs": round(gbs, 2),
        "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2), "decode_steps_per_s": round(1e3 / ms_per_step, 2),
        "step_bytes": int(step_bytes), "splits": run.splits, "partials": run.partials,
        "min_seq_len": run.min_len, "chunks": dict(zip(("lead_chunks", "lead_pages", "tail_pages"), run.chunks())),
        "plain_entry_point": {"call": plain_call, "chunks": dict(zip(("lead_chunks", "lead_pages", "tail_pages"),
                                                                     run.fk.decode_chunks(run.gc.layout, B, Hq,
                                                                                          run.gc.page_table.shape[1],
                                                                                          run.splits_req))),
                              "ms_per_step": round(t_plain, 5), "gbs": round(plain_gbs, 2),
                              "pct_of_peak_hbm": round(100.0 * plain_gbs / PEAK_HBM_GBS, 2)},
        "append": (None if not run.paged else "fused into the split kernel" if run.fused else "quantize_append"),
        "kernel_ms": {"append": round(t_append, 5), "decode_split": round(t_split, 5),
                      "decode_combine": round(t_comb, 5), "decode_split_back_to_back": round(t_split_b2b, 5)},
        "host_enqueue_ms_per_step": round(1e3 * host_enqueue / steps, 5), "wall_s_timed": round(wall, 4),
        "roofline": {"bound": "hbm", "kernel": run.split_kernel_name(), "achieved": round(split_gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(split_gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(w.name, run.fmt), "algorithmic_bytes_per_launch": int(split_bytes_b2b)},
    }


def cold_warm(torch, run, stream, reps=20):
    """For a cache smaller than the last-level cache: the step (one decode
    call, as DecodeRun.step makes it) cold (1 GiB of unrelated data read and
    written between calls, outside the timed events, so every call reads the
    cache from HBM; median of `reps`) and warm (back to back: the cache stays
    in the last-level cache), and the split kernel alone cold for the
    roofline block.  Steps this small take less GPU time than the host needs
    to enqueue them, so the warm calls queue behind a spin kernel that
    touches no memory and the cold ones behind the scrub: both time the GPU,
    not the host."""
    w = run.w
    B, Hq, D = w.batch, w.q_heads, w.head_dim
    ctx = [int(x) for x in run.lens0]
    split_bytes = run.split_bytes(ctx)
    step_bytes = split_bytes + B * Hq * D * 4
    scrub = torch.zeros(1 << 28, dtype=torch.int32, device=run.dev)     # 1 GiB
    for s in range(5):
        run.step(s)
    e0, e1 = _events(torch)
    torch.cuda.synchronize()
    torch.cuda._sleep(2_000_000)                  # ~1 ms of GPU clock cycles while the calls are enqueued
    e0.record(stream)
    for s in range(reps):
        run.step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    warm = e0.elapsed_time(e1) / reps

    def cold(call):
        times = []
        for s in range(reps):
            scrub.add_(1)
            c0, c1 = _events(torch)
            c0.record(stream)
            call(s)
            c1.record(stream)
            torch.cuda.synchronize()
            times.append(c0.elapsed_time(c1))
        return sorted(times)[len(times) // 2], min(times)

    cold_ms, cold_min = cold(run.step)
    split_ms, _ = cold(run.split)
    del scrub
    gbs = step_bytes / (cold_ms * 1e-3) / 1e9
    split_gbs = split_bytes / (split_ms * 1e-3) / 1e9
    return {
        "workload": w.name, "cache_bytes": run.gc.layout.cache_bytes, "step_bytes": int(step_bytes),
        "splits": run.splits, "partials": run.partials,
        "ms_per_step": round(cold_ms, 5), "gbs": round(gbs, 1), "pct_of_peak_hbm": round(100.0 * gbs / PEAK_HBM_GBS, 2),
        "decode_steps_per_s": round(1e3 / cold_ms, 2), "cold_ms_min": round(cold_min, 5),
        "warm_ms": round(warm, 5), "warm_gbs": round(step_bytes / (warm * 1e-3) / 1e9, 1),
        "warm_decode_steps_per_s": round(1e3 / warm, 2),
        "roofline": {"bound": "hbm", "kernel": run.split_kernel_name(), "achieved": round(split_gbs, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(split_gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic(w.name), "algorithmic_bytes_per_launch": int(split_bytes),
                     "split_cold_ms_median": round(split_ms, 5)},
        "note": "ms_per_step, gbs: cold (1 GiB scrubbed through the caches before each step, median of "
                f"{reps}); warm_*: back-to-back steps with the cache in the last-level cache",
    }


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
        ms = _time(torch, stream, call, reps)
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
    ap.add_argument("--splits", type=int, default=None,
                    help="context splits of the headline workload (default: the workload's)")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--format", choices=("fp4", "fp8", "fp8t"), default="fp4",
                    help="cache format: FP4 E2M1 + E4M3 per 16 (default), FP8 E4M3 with per-tensor scales, "
                         "or FP8 E4M3 with an fp16 scale per token (fp8t)")
    ap.add_argument("--unfused", action="store_true",
                    help="paged workload: append with quantize_append, then decode (default: the decode "
                         "kernel stores the new tokens itself)")
    ap.add_argument("--no-length-hint", action="store_true",
                    help="time the steps without the batch's shortest length (the plain entry points' chunking)")
    ap.add_argument("--kernel", choices=("auto", "mfma_staged", "mfma_direct", "valu"),
                    default="auto", help="split kernel of the timed steps (through fp4kv_decode_with_options "
                                         "unless auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-read-probe", action="store_true",
                    help="skip the streaming-read probe sweep (the achievable HBM read rate)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill quantise-append measurement (8 x 8192 tokens)")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only, not the other workloads")
    ap.add_argument("--config-steps", type=int, default=20, help="timed steps of each other workload")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the prefill quantise-append measurement (for profiling its kernel)")
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
    stream = torch.cuda.current_stream()

    if args.prefill_only:
        print(json.dumps({"prefill_append": prefill_append(fk, wl, args.seed, dev, stream)}), flush=True)
        return

    w = wl.WORKLOADS[args.workload]
    if w.kind == "prefill":
        raise SystemExit("the prefill workload is timed under configs (or alone with --prefill-only), "
                         "not as a decode step")
    run = DecodeRun(fk, hx, wl, w, args.seed, args.format, dev, args.warmup + args.steps, splits=args.splits,
                    unfused=args.unfused, kernel=args.kernel, length_hint=not args.no_length_hint)
    head = decode_record(torch, run, stream, args.steps, args.warmup)
    L = run.gc.layout
    result = {
        "metric": METRIC,
        "value": head["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "context": w.context if not run.paged else f"{w.min_len}..{w.max_len}",
                   "format": FORMAT_NAMES[args.format], "splits": run.splits, "partials": run.partials,
                   "page_size": 64, "cache_bytes": L.cache_bytes, "min_seq_len": head["min_seq_len"],
                   "chunks": head["chunks"]},
    }
    result.update({k: head[k] for k in ("decode_steps_per_s", "pct_of_peak_hbm", "append", "plain_entry_point")})
    result["kernel"] = args.kernel
    result.update({k: head[k] for k in ("kernel_ms", "wall_s_timed", "host_enqueue_ms_per_step")})
    result["settle_decode_calls"] = SETTLE_CALLS
    result["roofline"] = head["roofline"]
    if args.extras and not run.paged:
        result["extras"] = query_extras(fk, run.gc, w, dev, stream, run.splits_req)
    if L.cache_bytes < LLC_BYTES and not run.paged:
        result["cold_warm"] = cold_warm(torch, run, stream)
    cache_bytes = L.cache_bytes
    del run
    torch.cuda.empty_cache()
    if not args.no_read_probe:
        ceiling = read_ceiling(fk, dev, stream, cache_bytes)
        result["hbm_read_probe"] = ceiling
        result["roofline"]["frac_of_read_probe"] = round(result["roofline"]["achieved"] / ceiling["gbs"], 4)
        result["frac_of_read_probe"] = round(head["gbs"] / ceiling["gbs"], 4)
        torch.cuda.empty_cache()
    if not args.no_configs:
        configs = {}
        for name in SUB_CONFIGS:
            if name == w.name:
                continue
            cw = wl.WORKLOADS[name]
            r = DecodeRun(fk, hx, wl, cw, args.seed, "fp4", dev, args.warmup + args.config_steps,
                          length_hint=not args.no_length_hint)
            if r.gc.layout.cache_bytes < LLC_BYTES and not r.paged:
                configs[name] = cold_warm(torch, r, stream)
            else:
                configs[name] = decode_record(torch, r, stream, args.config_steps, args.warmup)
            del r
            torch.cuda.empty_cache()
        if not args.no_prefill:
            configs["prefill_b8_8k"] = prefill_append(fk, wl, args.seed, dev, stream)
            torch.cuda.empty_cache()
        result["configs"] = configs
    elif not args.no_prefill:
        result["prefill_append"] = prefill_append(fk, wl, args.seed, dev, stream)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        result["calibration_copy_bytes"] = src.numel()
        del src, dst
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, args.seed, oracle_threads(), args.format)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
