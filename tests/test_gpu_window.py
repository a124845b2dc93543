"""GPU parity of sliding-window attention over the packed cache
(fp4kv_decode_window_attention): query token i of S sees the last `window`
tokens of its causal prefix; each row within 1e-3 of the oracle's fp64
attention over exactly those tokens; window 0 is the unwindowed call."""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_harness as hx
import fp4kv_workloads as wl
import kv_formats as kf
import oracle
from test_gpu_multi_query import _cache

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _say(msg):
    print(msg, flush=True)


def _codes(kv, lens, fmt, L, D, Hkv):
    out = []
    for b, n in enumerate(lens):
        if fmt == "fp8t":
            out.append((kf.stored_values(fmt, L, kv[b][0]), kf.stored_values(fmt, L, kv[b][1])))
        elif fmt == "fp8":
            kc = oracle.quantize_fp8(wl.bf16_bits(kv[b][0]), L.params.k_scale) if n else np.zeros((1, Hkv, D), np.uint8)
            vc = oracle.quantize_fp8(wl.bf16_bits(kv[b][1]), L.params.v_scale) if n else np.zeros((1, Hkv, D), np.uint8)
            out.append((kc, vc))
        else:
            kq = oracle.quantize(wl.bf16_bits(kv[b][0]), want_xhat=False) if n else None
            vq = oracle.quantize(wl.bf16_bits(kv[b][1]), want_xhat=False) if n else None
            out.append((kq, vq))
    return out


def _reference(codes, lens, q, window, fmt, L, D, Hkv):
    """Oracle attention of query token i over tokens [lo_i, L_i)."""
    B, S, Hq, _ = q.shape
    ref = np.zeros((B, S, Hq, D))
    for b, n in enumerate(lens):
        for i in range(S):
            Li = n - (S - 1 - i)
            if Li <= 0:
                continue
            lo = max(0, Li - window) if window > 0 else 0
            qi = wl.bf16_bits(q[b:b + 1, i].contiguous())
            if fmt == "fp8t":
                kvals, vvals = codes[b]
                r = oracle.decode_attention_values(qi, [kvals[lo:Li]], [vvals[lo:Li]], [Li - lo], D ** -0.5)
            elif fmt == "fp8":
                kc, vc = codes[b]
                r = oracle.decode_attention_fp8(qi, [kc[lo:Li]], [vc[lo:Li]], L.params.k_scale, L.params.v_scale,
                                                [Li - lo], D ** -0.5)
            else:
                kq, vq = codes[b]
                r = oracle.decode_attention(qi, [kq[0][lo:Li]], [kq[1][lo:Li]], [vq[0][lo:Li]], [vq[1][lo:Li]],
                                            [Li - lo], D ** -0.5)
            ref[b, i] = r[0]
    return ref


@pytest.mark.parametrize("fmt,D", [("fp4", 128), ("fp4", 64), ("fp8", 128), ("fp8", 64), ("fp8t", 128),
                                   ("fp8t", 64)])
@pytest.mark.parametrize("window", [1, 17, 64, 100, 1000])
@pytest.mark.parametrize("S,G,splits", [(1, 8, 0), (4, 4, 1), (2, 2, 3)])
def test_window_against_oracle(fmt, D, window, S, G, splits):
    lens = [0, 1, 5, 64, 65, 200, 1000, 3000]
    Hkv = 2
    L, cache, table, kv, g = _cache(lens, Hkv, D, fmt, seed=window + S * 13 + D)
    q = torch.randn(len(lens), S, Hkv * G, D, generator=g).to(torch.bfloat16)
    _say(f"window attention: {fmt} D {D} window {window} S {S} G {G} splits {splits}")
    out = fk.decode_window_attention(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                                     table.cuda(), window, num_splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = _reference(_codes(kv, lens, fmt, L, D, Hkv), lens, q, window, fmt, L, D, Hkv)
    err = float(hx.row_rel_error(out, ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL


def test_window_zero_is_unwindowed():
    lens = [7, 130, 900]
    L, cache, table, kv, g = _cache(lens, 2, 128, "fp4", seed=4)
    q = torch.randn(3, 2, 8, 128, generator=g).to(torch.bfloat16)
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    a = fk.decode_window_attention(L, cache, q.cuda(), lens_d, table.cuda(), 0)
    b = fk.decode_multi_attention(L, cache, q.cuda(), lens_d, table.cuda())
    torch.cuda.synchronize()
    assert torch.equal(a, b)



def test_full_size_batch_multi_query_and_window():
    """The 32-sequence, 32768-token cache at its bench launch configuration:
    two query tokens per sequence in one pass (16 columns per KV head), and a
    4096-token window; sampled sequences against the oracle."""
    from test_gpu_decode import _oracle_decode
    w = wl.WORKLOADS["gqa8_b32_ctx32k"]
    seqs = [0, 31]
    gc = hx.build_cache(w, seed=1, keep_seqs=seqs)
    S = 2
    g = torch.Generator().manual_seed(12)
    q = torch.randn(w.batch, S, w.q_heads, w.head_dim, generator=g).to(torch.bfloat16)
    lens = gc.lens_cpu.tolist()
    scale = w.head_dim ** -0.5
    for window, splits in ((0, w.splits), (4096, 0)):
        _say(f"window attention: {w.name}, S {S}, window {window}, splits {splits}, oracle on {seqs}")
        out = fk.decode_window_attention(gc.layout, gc.cache, q.cuda(), gc.seq_lens, gc.page_table, window,
                                         num_splits=splits)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        for i in range(S):
            li = [n - (S - 1 - i) for n in lens]
            lo = [max(0, n - window) if window else 0 for n in li]
            kept = {b: (gc.kept[b][0][lo[b]:li[b]], gc.kept[b][1][lo[b]:li[b]]) for b in seqs}
            ref = _oracle_decode(q[:, i].contiguous(), kept, [li[b] - lo[b] for b in range(w.batch)], w.head_dim,
                                 scale)
            err = max(float(hx.row_rel_error(out[b, i], ref[b]).max()) for b in seqs)
            _say(f"  query token {i}: worst per-row relative error {err:.3e}")
            assert err <= TOL
