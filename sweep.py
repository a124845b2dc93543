"""Bit-width sweep on the GPU: attention-output error, cost and decode speed
of KV-cache formats on the seeded synthetic workloads.

The formats are the rows of the results table in "Quantising the KV cache"
(numerics-explained, Concept section): bf16 (the unquantised cache), FP8
E4M3 with one scale per tensor, INT8 per token, FP4 E2M1 with an E4M3 scale
per 16, INT4 and INT2 per token, and INT4 / INT2 with K per channel and V per
token; plus FP8 E4M3 with an fp16 scale per token, or K per channel and V per
token (the finer FP8 scale granularities of "KV Cache Quantisation", Common
questions).  The sweep itself is the lab of "Week 6 -- FP4 KV Caches and Bounded
Replay" (quantise synthetic KV at several bit widths and measure the
attention output's error).

Every step runs in the library's kernels: quantise-append and decode for FP4
and per-tensor FP8, int_quantize and int_decode_attention for bf16, the
integer formats and FP8 with per-token / per-channel scales.  For each format:
    row error = max_d |o - o_ref| / max_d |o_ref|   per (sequence, query head)
against the bf16 cache's output o_ref, and bits per number from the bytes
the format stores.  With --time, each format's decode is also timed on a
larger workload (inputs drawn on the GPU with the same distributions) and
its cache bytes per second reported, with the kernel that decodes it.
Every format decodes on the matrix cores: FP4 and per-tensor FP8 on the
product path's split-K kernels (paged cache), bf16, the integer formats and
FP8 with per-token / per-channel scales on the sweep's own split-K kernel
(contiguous rows), which turns each stored code into an exact bf16 operand
on the vector ALUs.  That conversion costs about the same per number at
every width, so the narrow formats (INT4, INT2) are bound by it rather than
by their few bytes: their rates fall below the 8-bit formats' while their
times stay close.

    python sweep.py                       # error table, 4096-token workload
    python sweep.py --workload tiny_d64_ctx256
    python sweep.py --time gqa8_b32_ctx32k
Prints the table on stderr and one JSON line on stdout.
"""
import argparse
import json
import math
import sys

import torch

import fp4_quantised_kv_amd as fk
import fp4kv_workloads as wl

# (name, kind, element bits, K granularity, V granularity)
FORMATS = [
    ("BF16, unquantised", "bf16", 16, "token", "token"),
    ("FP8 E4M3, one scale per tensor", "fp8", 8, None, None),
    ("FP8 E4M3 per token", "int", fk.INT_FP8_E4M3, "token", "token"),
    ("FP8 E4M3, K per channel, V per token", "int", fk.INT_FP8_E4M3, "channel", "token"),
    ("INT8 per token", "int", 8, "token", "token"),
    ("FP4 E2M1, E4M3 scale per 16", "fp4", 4, None, None),
    ("INT4 per token", "int", 4, "token", "token"),
    ("INT4, K per channel, V per token", "int", 4, "channel", "token"),
    ("INT2 per token", "int", 2, "token", "token"),
    ("INT2, K per channel, V per token", "int", 2, "channel", "token"),
]


class Prepared:
    """One format's stored K and V for a batch of equal-length sequences, and
    a decode call over them."""

    def __init__(self, kind, bits, kg, vg, k, v, scales):
        self.kind, self.bits, self.kg, self.vg = kind, bits, kg, vg
        B, T, H, D = k.shape
        self.B, self.T, self.H, self.D = B, T, H, D
        if kind in ("fp4", "fp8"):
            pages = -(-T // fk.PAGE_SIZE)
            if kind == "fp8":
                self.layout = fk.cache_layout(H, D, B * pages, format=fk.FORMAT_FP8_E4M3,
                                              k_scale=scales[0], v_scale=scales[1])
            else:
                self.layout = fk.cache_layout(H, D, B * pages)
            self.cache = torch.zeros(self.layout.cache_bytes, dtype=torch.uint8, device=k.device)
            slots = torch.arange(B * pages * fk.PAGE_SIZE, device=k.device).view(B, -1)[:, :T].reshape(-1)
            fk.quantize_append(self.layout, k.reshape(B * T, H, D), v.reshape(B * T, H, D),
                               slots.contiguous(), self.cache)
            self.table = torch.arange(B * pages, dtype=torch.int32, device=k.device).view(B, pages)
            self.lens = torch.full((B,), T, dtype=torch.int32, device=k.device)
            self.stored_bytes = B * T * self.layout.bytes_per_token
        else:
            self.kq = fk.int_quantize(k, bits, kg)
            self.vq = fk.int_quantize(v, bits, vg)
            self.stored_bytes = sum(t.numel() * t.element_size() for t in (*self.kq, *self.vq))
        self.bits_per_number = 8.0 * self.stored_bytes / (2 * B * T * H * D)
        if kind == "fp8":
            self.bits_per_number = 8.0                  # the two per-tensor fp32 scales are kept outside

    def decode(self, q, workspace=None, out=None):
        if self.kind in ("fp4", "fp8"):
            return fk.decode_attention(self.layout, self.cache, q, self.lens, self.table,
                                       workspace=workspace, out=out)
        return fk.int_decode_attention(q, self.bits, self.kq, self.vq, self.T, self.kg, self.vg,
                                       workspace=workspace, out=out)

    def workspace_bytes(self, Hq):
        if self.kind in ("fp4", "fp8"):
            return fk.decode_plan(self.layout, self.B, Hq, self.table.shape[1], 0).workspace_bytes
        return fk.int_decode_plan(self.B, self.T, self.H, self.D, Hq, 0)[1]


def supported(kind, head_dim):
    """Every format is built for head dims 64 and 128."""
    return head_dim in (64, 128)


def row_errors(out, ref):
    num = (out.double() - ref.double()).abs().amax(dim=-1)
    den = ref.double().abs().amax(dim=-1)
    return (num / den).flatten()


def error_table(name, seed, device="cuda"):
    """Rows (format, bits per number, mean row error, max row error) for a
    seeded workload whose sequences all hold w.context tokens."""
    w = wl.WORKLOADS[name]
    T = w.context
    k = torch.stack([wl.kv_tokens(w, seed, b, "k", 0, T) for b in range(w.batch)]).to(device)
    v = torch.stack([wl.kv_tokens(w, seed, b, "v", 0, T) for b in range(w.batch)]).to(device)
    q = wl.queries(w, seed).to(device)
    scales = wl.fp8_tensor_scales(w, seed)
    outs, bpn = {}, {}
    for fname, kind, bits, kg, vg in FORMATS:
        if not supported(kind, w.head_dim):
            continue
        p = Prepared(kind, bits, kg, vg, k, v, scales)
        outs[fname] = p.decode(q)
        bpn[fname] = p.bits_per_number
        del p
    torch.cuda.synchronize()
    ref = outs[FORMATS[0][0]]
    rows = []
    for fname, *_ in FORMATS:
        if fname not in outs:
            rows.append((fname, None, None, None))
            continue
        e = row_errors(outs[fname], ref)
        rows.append((fname, bpn[fname], float(e.mean()), float(e.max())))
    return rows


def synthetic_gpu(w, seed, device):
    """K, V [B][T][H][D] and q drawn on the GPU with the workload's
    distributions (its channel factors), for timing only."""
    g = torch.Generator(device=device).manual_seed(seed)
    fk_, fv_ = wl.channel_factors(w, seed, "k").to(device), wl.channel_factors(w, seed, "v").to(device)
    shape = (w.batch, w.context, w.kv_heads, w.head_dim)
    k = (torch.randn(shape, generator=g, device=device) * fk_).to(torch.bfloat16)
    v = (torch.randn(shape, generator=g, device=device) * fv_).to(torch.bfloat16)
    q = torch.randn(w.batch, w.q_heads, w.head_dim, generator=g, device=device).to(torch.bfloat16)
    return k, v, q


def timing_table(name, seed, reps, device="cuda"):
    """Per format: decode ms (mean of `reps` back-to-back calls) and the
    achieved rate over the bytes it must read (stored K and V, q, out)."""
    w = wl.WORKLOADS[name]
    k, v, q = synthetic_gpu(w, seed, device)
    scales = wl.fp8_tensor_scales(w, seed)
    rows = []
    for fname, kind, bits, kg, vg in FORMATS:
        if not supported(kind, w.head_dim):
            continue
        p = Prepared(kind, bits, kg, vg, k, v, scales)
        ws = torch.empty(max(p.workspace_bytes(w.q_heads), 256), dtype=torch.uint8, device=device)
        out = torch.empty(w.batch, w.q_heads, w.head_dim, dtype=torch.float32, device=device)
        for _ in range(3):
            p.decode(q, ws, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            p.decode(q, ws, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        nbytes = p.stored_bytes + q.numel() * 2 + out.numel() * 4
        kernel = "matrix-core split-K, paged" if kind in ("fp4", "fp8") else "matrix-core split-K, sweep formats"
        rows.append((fname, p.bits_per_number, ms, nbytes / (ms * 1e-3) / 1e9, kernel))
        print(f"# timed {fname}: {ms:.4f} ms", file=sys.stderr, flush=True)
        del p, ws, out
        torch.cuda.empty_cache()
    return rows


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--workload", default="gqa4_b8_ctx4k", help="workload for the error table")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--time", default=None, help="also time every format's decode on this workload")
    ap.add_argument("--reps", type=int, default=20)
    args = ap.parse_args()
    if not torch.cuda.is_available():
        sys.exit("sweep.py needs a GPU")
    w = wl.WORKLOADS[args.workload]
    if w.kind != "decode":
        sys.exit("the sweep needs a workload of equal-length sequences")
    rows = error_table(args.workload, args.seed)
    print(f"# {args.workload} (seed {args.seed}): {w.description}", file=sys.stderr)
    print(f"# {'format':36s} {'bits/number':>11s} {'mean row err':>13s} {'max row err':>12s}", file=sys.stderr)
    for r in rows:
        if r[1] is None:
            print(f"  {r[0]:36s} {'(not built for this head size)':>38s}", file=sys.stderr)
        else:
            print(f"  {r[0]:36s} {r[1]:11.4f} {r[2]:13.4e} {r[3]:12.4e}", file=sys.stderr)
    result = {"sweep": "attention-output error vs bits per number", "workload": args.workload,
              "seed": args.seed, "reference": FORMATS[0][0],
              "rows": [{"format": r[0], "bits_per_number": None if r[1] is None else round(r[1], 6),
                        "mean_row_error": r[2], "max_row_error": r[3]} for r in rows]}
    if args.time:
        t = timing_table(args.time, args.seed, args.reps)
        result["timing"] = {"workload": args.time, "reps": args.reps,
                            "note": "every format decodes on the matrix cores ('kernel': the paged "
                                    "product kernels or the sweep formats' kernel); the narrow integer "
                                    "formats are bound by converting codes to operands, not by bytes",
                            "rows": [{"format": r[0], "bits_per_number": round(r[1], 6), "kernel": r[4],
                                      "decode_ms": round(r[2], 5), "gbs": round(r[3], 1),
                                      "pct_of_peak_hbm": round(100.0 * r[3] / 8000.0, 1)} for r in t]}
        print(f"# decode on {args.time} (INT4 / INT2: bound by converting codes to matrix-core operands)",
              file=sys.stderr)
        for r in t:
            print(f"  {r[0]:36s} {r[1]:8.4f} bits  {r[2]:9.4f} ms  {r[3]:8.1f} GB/s  {100.0 * r[3] / 8000.0:5.1f} %  "
                  f"{r[4]}", file=sys.stderr)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
