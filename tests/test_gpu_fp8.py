"""GPU parity of the FP8 E4M3 (one scale per tensor) cache: stored bytes
bit-exact against the oracle's codes, decode attention within 1e-3 per row
of the oracle's fp64 attention over the same codes."""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_harness as hx
import fp4kv_workloads as wl
import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _say(msg):
    print(msg, flush=True)


def _layout(H, pages, ks, vs, D=128):
    return fk.cache_layout(H, D, pages, format=fk.FORMAT_FP8_E4M3, k_scale=ks, v_scale=vs)


def _to_rows(bits, H=1, D=128):
    """uint16 [n] bf16 patterns -> bf16 tensor [n_tok][H][D] (zero padded)."""
    per = H * D
    n_tok = -(-bits.size // per)
    pad = np.zeros(n_tok * per, np.uint16)
    pad[: bits.size] = bits
    return torch.from_numpy(pad.view(np.int16).reshape(n_tok, H, D)).view(torch.bfloat16)


def _append_and_read(k, v, ks, vs, slots=None):
    n, H, D = k.shape
    if slots is None:
        slots = torch.arange(n, dtype=torch.int64)
    pages = int(slots.max()) // 64 + 1 if n else 1
    L = _layout(H, pages, ks, vs, D)
    cache = torch.zeros(L.cache_bytes, dtype=torch.uint8, device="cuda")
    fk.quantize_append(L, k.cuda(), v.cuda(), slots.cuda(), cache)
    torch.cuda.synchronize()
    return L, cache


@pytest.mark.parametrize("ks,vs,D", [(1.0, 0.75, 128), (0.0173, 3.3, 128), (2.0 ** -20, 123.456, 128),
                                     (1.0 / 7.0, 2.0 ** 10, 128), (0.0173, 3.3, 64)])
def test_every_bf16_value(ks, vs, D):
    """Every finite bf16 pattern as K (in order) and V (reversed), under
    general fp32 scales, power-of-two scales and scales that put quotients
    exactly on E4M3 rounding midpoints."""
    allb = np.array([b for b in range(0x10000) if (b >> 7) & 0xFF != 0xFF], np.uint16)
    k = _to_rows(allb, D=D)
    v = _to_rows(allb[::-1].copy(), D=D)
    _say(f"fp8 quantize_append: every bf16, scales {ks}, {vs}, {k.shape[0]} tokens")
    L, cache = _append_and_read(k, v, ks, vs)
    kc, vc = hx.read_pages_fp8(cache, L, list(range(L.num_pages)), k.shape[0])
    assert np.array_equal(kc, oracle.quantize_fp8(wl.bf16_bits(k), L.params.k_scale))
    assert np.array_equal(vc, oracle.quantize_fp8(wl.bf16_bits(v), L.params.v_scale))


def test_scattered_slots_and_skips():
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    k = wl.kv_tokens(w, 6, 0, "k", 0, 300)
    v = wl.kv_tokens(w, 6, 0, "v", 0, 300)
    perm = torch.randperm(640, generator=torch.Generator().manual_seed(1))[:300].to(torch.int64)
    slots = perm.clone()
    slots[::37] = -1                                   # skipped
    _say("fp8 quantize_append: 300 tokens at scattered slots, some skipped")
    L = _layout(w.kv_heads, 10, 0.05, 0.02)
    cache = torch.full((L.cache_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    fk.quantize_append(L, k.cuda(), v.cuda(), slots.cuda(), cache)
    torch.cuda.synchronize()
    kc, vc = hx.read_pages_fp8(cache, L, list(range(10)), 640)
    ek = oracle.quantize_fp8(wl.bf16_bits(k), L.params.k_scale)
    ev = oracle.quantize_fp8(wl.bf16_bits(v), L.params.v_scale)
    written = set()
    for t, s in enumerate(slots.tolist()):
        if s >= 0:
            assert np.array_equal(kc[s], ek[t]) and np.array_equal(vc[s], ev[t])
            written.add(s)
    for s in range(640):
        if s not in written:
            assert (kc[s] == 0x5A).all() and (vc[s] == 0x5A).all()


def _decode_ref(q, kept, lens, ks, vs, scale, Hkv, D=128):
    kcodes, vcodes = [], []
    for b in range(len(lens)):
        k, v = kept[b]
        kcodes.append(oracle.quantize_fp8(wl.bf16_bits(k[: lens[b]]), ks).reshape(-1, Hkv, D)
                      if lens[b] else np.zeros((0, Hkv, D), np.uint8))
        vcodes.append(oracle.quantize_fp8(wl.bf16_bits(v[: lens[b]]), vs).reshape(-1, Hkv, D)
                      if lens[b] else np.zeros((0, Hkv, D), np.uint8))
    return oracle.decode_attention_fp8(wl.bf16_bits(q), kcodes, vcodes, ks, vs, lens, scale)


@pytest.mark.parametrize("G", [1, 3, 8, 16])
@pytest.mark.parametrize("splits", [0, 1, 5])
@pytest.mark.parametrize("D", [128, 64])
def test_decode_ragged_lengths(G, splits, D):
    """Lengths 0, 1, 31, 32, 33, 63, 64, 65, 1000 (empty rows, both halves of
    a page ragged), random page order, garbage in never-written slots."""
    lens = [0, 1, 31, 32, 33, 63, 64, 65, 1000]
    Hkv = 2
    g = torch.Generator().manual_seed(40 + G)
    maxp = max(-(-l // 64) for l in lens)
    table = torch.randperm(len(lens) * maxp, generator=g).to(torch.int32).reshape(len(lens), maxp)
    L = _layout(Hkv, len(lens) * maxp, 0.04, 0.015, D)
    cache = torch.full((L.cache_bytes,), 0x7F, dtype=torch.uint8, device="cuda")   # NaN codes
    kept = {}
    for b, n in enumerate(lens):
        k = (torch.randn(n, Hkv, D, generator=g) * 3.0).to(torch.bfloat16)
        v = torch.randn(n, Hkv, D, generator=g).to(torch.bfloat16)
        kept[b] = (k, v)
        if n:
            fk.quantize_append(L, k.cuda(), v.cuda(), wl.slots_for(table, b, 0, n).cuda(), cache)
    q = torch.randn(len(lens), G * Hkv, D, generator=g).to(torch.bfloat16)
    _say(f"fp8 decode: ragged lens {lens}, G={G}, splits={splits}, D={D}")
    out = fk.decode_attention(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                              table.cuda(), num_splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = _decode_ref(q, kept, lens, L.params.k_scale, L.params.v_scale, D ** -0.5, Hkv, D)
    assert np.array_equal(out[0], np.zeros_like(out[0]))
    err = hx.row_rel_error(out[1:], ref[1:])
    _say(f"  worst per-row relative error {float(err.max()):.3e}")
    assert float(err.max()) <= TOL


@pytest.mark.parametrize("name,seqs", [("gqa4_b8_ctx4k", None), ("gqa8_b32_ctx32k", [0, 31]),
                                       ("paged_b64_len1k_16k", [0, 17, 63])])
def test_decode_workloads(name, seqs):
    """Whole small workload, or sampled sequences of the 32K batch and the
    paged pool at their benchmark launch configuration."""
    w = wl.WORKLOADS[name]
    keep = range(w.batch) if seqs is None else seqs
    _say(f"fp8 decode: {name}, checking sequences {list(keep)}")
    gc = hx.build_cache(w, seed=2, keep_seqs=keep, fmt="fp8", zero=False)
    q = wl.queries(w, 2)
    out = fk.decode_attention(gc.layout, gc.cache, q.cuda(), gc.seq_lens, gc.page_table,
                              num_splits=w.splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    lens = gc.lens_cpu.tolist()
    Hkv = w.kv_heads
    kc, vc = [], []
    for b in range(w.batch):
        if b in gc.kept:
            k, v = gc.kept[b]
            kc.append(oracle.quantize_fp8(wl.bf16_bits(k), gc.layout.params.k_scale))
            vc.append(oracle.quantize_fp8(wl.bf16_bits(v), gc.layout.params.v_scale))
        else:
            kc.append(np.zeros((1, Hkv, 128), np.uint8))
            vc.append(np.zeros((1, Hkv, 128), np.uint8))
    heads = [(b, h) for b in keep for h in range(Hkv)]
    ref = oracle.decode_attention_fp8(wl.bf16_bits(q), kc, vc, gc.layout.params.k_scale,
                                      gc.layout.params.v_scale, lens, 128 ** -0.5, heads=heads)
    err = max(float(hx.row_rel_error(out[b], ref[b]).max()) for b in keep)
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL
    # stored bytes of the checked sequences, too
    for b in list(keep)[:2]:
        n = lens[b]
        kb, vb = hx.read_pages_fp8(gc.cache, gc.layout, gc.pt_cpu.table[b, : -(-n // 64)].tolist(), n)
        assert np.array_equal(kb, kc[b]) and np.array_equal(vb, vc[b])
