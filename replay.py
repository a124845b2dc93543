"""Exact versus bounded replay of sliding-window state, on the GPU.

"Week 6 -- FP4 KV Caches and Bounded Replay" (Overview, Core Concepts,
Lecture notes, Lab): sliding-window (SWA) layers attend over the last n_win
tokens; rebuilding every layer's window exactly means replaying about
L * n_win tokens, bounded replay replays only the last n_win tokens and pays
a small error.  This script measures both in a toy network of L SWA layers
with random weights (fp4kv_workloads.TOY_NETS), its K/V windows held in the
library's FP8 (one scale per tensor) or FP4 cache:

  reference       the last token's output after running all tokens;
  exact replay    the same from empty windows over the last L*(n_win-1)+1
                  tokens -- identical to the reference, bit for bit;
  bounded replay  the same over the last n_win tokens only.

Each token step runs, per layer, the projections (plain GEMMs through
torch), quantize_append of the token's K and V into the layer's cache and
decode_window_attention over its last n_win tokens.  Reports the bounded
replay's relative error ||y - y_ref|| / ||y_ref||, the tokens each replay
processes (the compute saved) and their GPU time.

    python replay.py [--net toy_swa_l4_w32] [--format fp8|fp4] [--curve]
Prints a table on stderr and one JSON line on stdout.
"""
import argparse
import json
import sys
import time

import torch

import fp4_quantised_kv_amd as fk
import fp4kv_workloads as wl

FP8_SCALE = 6.0 / 448.0          # a 6-sigma value of a unit-variance channel at the top of E4M3


class ToySwaGpu:
    """The toy network with its K/V windows in the library's cache."""

    def __init__(self, net: wl.ToyNet, weights, fmt: str, device="cuda"):
        self.net, self.fmt, self.device = net, fmt, device
        self.w = [tuple(m.to(device) for m in layer) for layer in weights]
        self.pages_per_seq = -(-net.tokens // fk.PAGE_SIZE)
        pages = net.batch * self.pages_per_seq
        if fmt == "fp8":
            self.layout = fk.cache_layout(net.kv_heads, net.head_dim, pages, format=fk.FORMAT_FP8_E4M3,
                                          k_scale=FP8_SCALE, v_scale=FP8_SCALE)
        elif fmt == "fp4":
            self.layout = fk.cache_layout(net.kv_heads, net.head_dim, pages)
        else:
            raise ValueError("format is fp8 or fp4")
        self.table = torch.arange(pages, dtype=torch.int32, device=device).view(net.batch, -1)
        # token position p of sequence b lives in slot b * pages_per_seq * 64 + p, in every run, so
        # that a replay lays its tokens out exactly as the full run does
        self.seq_base = torch.arange(net.batch, dtype=torch.int64, device=device) * self.pages_per_seq * fk.PAGE_SIZE

    def run(self, x: torch.Tensor, start: int, end: int, record=None) -> torch.Tensor:
        """Final hidden states of tokens start .. end-1 ([B][end-start][d],
        fp32), from empty windows.  With a list `record`, appends for every
        token the (q, k, v) bf16 rows and the attention output of each layer
        (CPU copies), then the layers' caches."""
        net = self.net
        B, Hq, Hkv, D = net.batch, net.q_heads, net.kv_heads, net.head_dim
        caches = [torch.zeros(self.layout.cache_bytes, dtype=torch.uint8, device=self.device)
                  for _ in range(net.layers)]
        out = torch.empty(B, end - start, net.d_model, dtype=torch.float32, device=self.device)
        for t in range(start, end):
            h = x[:, t]
            slots = self.seq_base + t
            lens = torch.full((B,), t + 1, dtype=torch.int32, device=self.device)
            window = min(net.window, t - start + 1)          # no token before `start` exists
            for layer, (wq, wk, wv, wo) in enumerate(self.w):
                u = h * torch.rsqrt(torch.mean(h * h, dim=1, keepdim=True))
                q = (u @ wq).to(torch.bfloat16).view(B, 1, Hq, D)
                k = (u @ wk).to(torch.bfloat16).view(B, Hkv, D)
                v = (u @ wv).to(torch.bfloat16).view(B, Hkv, D)
                fk.quantize_append(self.layout, k, v, slots, caches[layer])
                attn = fk.decode_window_attention(self.layout, caches[layer], q, lens, self.table, window)
                if record is not None:
                    if layer == 0:
                        record.append([])
                    record[-1].append((q.view(B, Hq, D).cpu(), k.cpu(), v.cpu(), attn.view(B, Hq, D).cpu()))
                h = h + attn.view(B, Hq * D) @ wo
            out[:, t - start] = h
        if record is not None:
            record.append([c.cpu() for c in caches])
        return out


def replay_lengths(net: wl.ToyNet):
    return net.layers * (net.window - 1) + 1, net.window


def relative_errors(a, ref):
    return (torch.linalg.vector_norm((a - ref).double(), dim=-1) /
            torch.linalg.vector_norm(ref.double(), dim=-1))


def study(name: str, seed: int, fmt: str, device="cuda"):
    """(reference, exact replay, bounded replay) outputs of the last token
    [B][d], and the GPU milliseconds of the three runs."""
    net = wl.TOY_NETS[name]
    gpu = ToySwaGpu(net, wl.toy_weights(net, seed), fmt, device)
    x = wl.toy_inputs(net, seed).to(device)
    N = net.tokens
    r_exact, r_bounded = replay_lengths(net)
    outs, ms = [], []
    for start in (0, N - r_exact, N - r_bounded):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        y = gpu.run(x, start, N)[:, -1]
        e1.record()
        torch.cuda.synchronize()
        outs.append(y)
        ms.append(e0.elapsed_time(e1))
    return outs, ms


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--net", default="toy_swa_l4_w32", choices=sorted(wl.TOY_NETS))
    ap.add_argument("--format", default="fp8", choices=("fp8", "fp4"))
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--curve", action="store_true",
                    help="also the error after replaying window, 2*window, ... tokens (quality vs compute)")
    args = ap.parse_args()
    if not torch.cuda.is_available():
        sys.exit("replay.py needs a GPU")
    net = wl.TOY_NETS[args.net]
    t0 = time.perf_counter()
    (ref, exact, bounded), ms = study(args.net, args.seed, args.format)
    r_exact, r_bounded = replay_lengths(net)
    e_exact = relative_errors(exact, ref)
    e_bounded = relative_errors(bounded, ref)
    result = {
        "study": "exact vs bounded replay of sliding-window KV state", "net": args.net, "seed": args.seed,
        "layers": net.layers, "window": net.window, "batch": net.batch, "tokens": net.tokens,
        "kv_format": args.format,
        "exact_replay": {"tokens": r_exact, "gpu_ms": round(ms[1], 3), "bit_identical": bool(torch.equal(exact, ref)),
                         "max_rel_error": float(e_exact.max())},
        "bounded_replay": {"tokens": r_bounded, "gpu_ms": round(ms[2], 3),
                           "mean_rel_error": float(e_bounded.mean()), "max_rel_error": float(e_bounded.max())},
        "full_run": {"tokens": net.tokens, "gpu_ms": round(ms[0], 3)},
        "compute_saved": round(r_exact / r_bounded, 3),
        "wall_s": round(time.perf_counter() - t0, 2),
    }
    if args.curve:
        gpu = ToySwaGpu(net, wl.toy_weights(net, args.seed), args.format)
        x = wl.toy_inputs(net, args.seed).to("cuda")
        points = []
        for r in list(range(net.window, r_exact, net.window)) + [r_exact]:
            y = gpu.run(x, net.tokens - r, net.tokens)[:, -1]
            points.append({"tokens": r, "mean_rel_error": float(relative_errors(y, ref).mean())})
        result["curve"] = points
        for pt in points:
            print(f"  replay {pt['tokens']:5d} tokens: error {pt['mean_rel_error']:.3e}", file=sys.stderr)
    print(f"# {args.net} ({net.layers} layers, window {net.window}, {args.format} K/V), batch {net.batch}",
          file=sys.stderr)
    print(f"  exact replay   {r_exact:5d} tokens  {ms[1]:8.2f} ms  error {float(e_exact.max()):.3e}"
          f"  identical: {result['exact_replay']['bit_identical']}", file=sys.stderr)
    print(f"  bounded replay {r_bounded:5d} tokens  {ms[2]:8.2f} ms  error mean {float(e_bounded.mean()):.3e}"
          f" max {float(e_bounded.max()):.3e}", file=sys.stderr)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
