"""Writes tests/golden/bitwidth_sweep_<workload>.txt from the oracle alone.

The bit-width sweep of "Week 6 -- FP4 KV Caches and Bounded Replay" (Lab
section: quantise synthetic KV at several bit widths and measure the
attention output's error) over the formats of the results table in
"Quantising the KV cache" (Concept section).  For each format the seeded
workload's K and V are quantised, attention of the workload's queries is
computed in fp64 over the stored values, and compared row by row with fp64
attention over the unquantised bf16 K and V:
    row error = max_d |o - o_ref| / max_d |o_ref|   per (sequence, query head)
The file lists bits per number (b + s/g as the layout stores it), the mean
and the largest row error.  Only oracle/ computes; run from the repository
root:  python tests/golden/make_bitwidth_sweep.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import fp4kv_workloads as wl  # noqa: E402
import oracle  # noqa: E402

# (name, kind, element bits, K granularity, V granularity)
FORMATS = [
    ("BF16, unquantised", "bf16", 16, None, None),
    ("FP8 E4M3, one scale per tensor", "fp8", 8, None, None),
    ("FP8 E4M3 per token", "fp8g", 8, "token", "token"),
    ("FP8 E4M3, K per channel, V per token", "fp8g", 8, "channel", "token"),
    ("INT8 per token", "int", 8, "token", "token"),
    ("FP4 E2M1, E4M3 scale per 16", "fp4", 4, None, None),
    ("INT4 per token", "int", 4, "token", "token"),
    ("INT4, K per channel, V per token", "int", 4, "channel", "token"),
    ("INT2 per token", "int", 2, "token", "token"),
    ("INT2, K per channel, V per token", "int", 2, "channel", "token"),
]
WORKLOADS = [("tiny_d64_ctx256", 1), ("gqa4_b8_ctx4k", 2)]


def bits_per_number(kind, bits, kg, vg, T, D):
    if kind == "bf16":
        return 16.0
    if kind == "fp8":
        return 8.0                               # two per-tensor scales: nothing per number
    if kind == "fp4":
        return oracle.bits_per_number(4, 8, 16)
    per = lambda g: oracle.bits_per_number(bits, 16, D if g == "token" else T)
    return (per(kg) + per(vg)) / 2


def stored_values(kind, bits, gran, x_bits, tensor_scale):
    """float64 [T][H][D] of one sequence's K or V as the format stores it."""
    if kind == "bf16":
        return oracle.bf16_values(x_bits)
    if kind == "fp8":
        return oracle.dequantize_fp8(oracle.quantize_fp8(x_bits, tensor_scale), tensor_scale)
    if kind == "fp4":
        return oracle.quantize(x_bits)[2]
    if kind == "fp8g":
        c, s = oracle.quantize_fp8_groups(x_bits, gran)
        return oracle.dequantize_fp8_groups(c, s, gran)
    c, s = oracle.quantize_int(x_bits, bits, gran)
    return oracle.dequantize_int(c, s, gran)


def row_errors(out, ref):
    num = np.max(np.abs(out - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return (num / den).ravel()


def sweep(name, seed):
    w = wl.WORKLOADS[name]
    T = w.context
    ks, vs = wl.fp8_tensor_scales(w, seed)
    kb = [wl.bf16_bits(wl.kv_tokens(w, seed, b, "k", 0, T)) for b in range(w.batch)]
    vb = [wl.bf16_bits(wl.kv_tokens(w, seed, b, "v", 0, T)) for b in range(w.batch)]
    q = wl.bf16_bits(wl.queries(w, seed))
    scale = w.head_dim ** -0.5
    lens = [T] * w.batch
    outs = {}
    for fname, kind, bits, kg, vg in FORMATS:
        kv = [stored_values(kind, bits, kg, kb[b], ks) for b in range(w.batch)]
        vv = [stored_values(kind, bits, vg, vb[b], vs) for b in range(w.batch)]
        outs[fname] = oracle.decode_attention_values(q, kv, vv, lens, scale)
    ref = outs[FORMATS[0][0]]
    rows = []
    for fname, kind, bits, kg, vg in FORMATS:
        e = row_errors(outs[fname], ref)
        rows.append((fname, bits_per_number(kind, bits, kg, vg, T, w.head_dim), float(e.mean()), float(e.max())))
    return w, rows


def main():
    for name, seed in WORKLOADS:
        w, rows = sweep(name, seed)
        path = os.path.join(HERE, f"bitwidth_sweep_{name}.txt")
        with open(path, "w") as f:
            f.write(f"# Bit-width sweep on the seeded {name} workload (seed {seed}): {w.description}\n")
            f.write("# Written by tests/golden/make_bitwidth_sweep.py from the oracle alone (fp64 attention\n")
            f.write("#   over each format's stored values against fp64 attention over the bf16 K and V).\n")
            f.write("# Formats: \"Quantising the KV cache\", Concept section, results table (the FP8 rows with\n")
            f.write("#   an fp16 scale per token / channel: \"KV Cache Quantisation\", Common questions); sweep: \"Week 6 --\n")
            f.write("#   FP4 KV Caches and Bounded Replay\", Lab section.  Row error = max_d |o - o_ref| /\n")
            f.write("#   max_d |o_ref| per (sequence, query head).\n")
            f.write("# format | bits per number | mean row error | max row error\n")
            for fname, bpn, mean, mx in rows:
                f.write(f"{fname} | {bpn:.6f} | {mean:.9e} | {mx:.9e}\n")
        print(path)
        for r in rows:
            print(f"  {r[0]:36s} {r[1]:8.4f} {r[2]:.3e} {r[3]:.3e}")


if __name__ == "__main__":
    main()
