"""GPU parity of the paged FP8 E4M3 cache with one fp16 scale per (token, KV
head): stored codes and scales bit-exact against the oracle's, decode
attention within 1e-3 per row of the oracle's fp64 attention over the same
stored values."""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_harness as hx
import fp4kv_workloads as wl
import kv_formats as kf
import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _say(msg):
    print(msg, flush=True)


def _to_rows(bits, H=1, D=128):
    per = H * D
    n_tok = -(-bits.size // per)
    pad = np.zeros(n_tok * per, np.uint16)
    pad[: bits.size] = bits
    return torch.from_numpy(pad.view(np.int16).reshape(n_tok, H, D)).view(torch.bfloat16)


def _check_bytes(cache, L, pages, n, k, v, slots=None):
    """Codes and scales of tokens k, v [n][H][D] against the oracle's; with
    `slots`, token t sits at slots[t] of the page list."""
    kc, vc = hx.read_pages_fp8(cache, L, pages, len(pages) * 64)
    ksc, vsc = hx.read_token_scales(cache, L, pages, len(pages) * 64)
    ek, eks = oracle.quantize_fp8_groups(wl.bf16_bits(k), "token")
    ev, evs = oracle.quantize_fp8_groups(wl.bf16_bits(v), "token")
    at = np.arange(n) if slots is None else np.asarray(slots)
    keep = at >= 0
    assert np.array_equal(kc[at[keep]], ek[keep]) and np.array_equal(ksc[at[keep]], eks[keep])
    assert np.array_equal(vc[at[keep]], ev[keep]) and np.array_equal(vsc[at[keep]], evs[keep])
    return kc, vc, ksc, vsc


@pytest.mark.parametrize("D", [128, 64])
def test_every_bf16_value(D):
    """Every finite bf16 pattern as K (in order) and V (reversed), D to a
    token row: every scale range (the 2^-24 fallback, normal, saturated at
    65504) and every element under them."""
    allb = np.array([b for b in range(0x10000) if (b >> 7) & 0xFF != 0xFF], np.uint16)
    k = _to_rows(allb, D=D)
    v = _to_rows(allb[::-1].copy(), D=D)
    n = k.shape[0]
    pages = -(-n // 64)
    L = kf.layout("fp8t", 1, D, pages)
    cache = torch.zeros(L.cache_bytes, dtype=torch.uint8, device="cuda")
    _say(f"fp8 per-token quantize_append: every bf16, D {D}, {n} tokens")
    fk.quantize_append(L, k.cuda(), v.cuda(), torch.arange(n, dtype=torch.int64).cuda(), cache)
    torch.cuda.synchronize()
    _check_bytes(cache, L, list(range(pages)), n, k, v)


def test_layout_sizes():
    L = kf.layout("fp8t", 8, 128, 3)
    assert L.block_bytes == 128 * 128 + 256
    assert L.k_scales_offset == 64 * 128 and L.v_codes_offset == 64 * 128 + 128
    assert L.v_scales_offset == 128 * 128 + 128
    assert L.bytes_per_token == 2 * 8 * (128 + 2)
    assert L.fp8 and L.token_scales


def test_scattered_slots_and_skips():
    """300 tokens of 8 KV heads at scattered slots, some skipped; the
    never-written slots keep their bytes."""
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    k = wl.kv_tokens(w, 6, 0, "k", 0, 300)
    v = wl.kv_tokens(w, 6, 0, "v", 0, 300)
    slots = torch.randperm(640, generator=torch.Generator().manual_seed(1))[:300].to(torch.int64)
    slots[::37] = -1
    _say("fp8 per-token quantize_append: 300 tokens at scattered slots, some skipped")
    L = kf.layout("fp8t", w.kv_heads, 128, 10)
    cache = torch.full((L.cache_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    fk.quantize_append(L, k.cuda(), v.cuda(), slots.cuda(), cache)
    torch.cuda.synchronize()
    kc, vc, ksc, vsc = _check_bytes(cache, L, list(range(10)), 300, k, v, slots.tolist())
    written = set(s for s in slots.tolist() if s >= 0)
    for s in range(640):
        if s not in written:
            assert (kc[s] == 0x5A).all() and (vc[s] == 0x5A).all()
            assert (ksc[s] == 0x5A5A).all() and (vsc[s] == 0x5A5A).all()


def _fill(lens, Hkv, D, seed, v_spread=0.0, fill=0x7F):
    """A cache of random page order holding lens[b] tokens per sequence
    (0x7F: NaN codes and NaN scales in never-written slots).  v_spread > 0
    gives every V token its own magnitude, log-uniform over e^[-v_spread,
    v_spread]."""
    g = torch.Generator().manual_seed(seed)
    maxp = max(1, max(-(-n // 64) for n in lens))
    table = torch.randperm(len(lens) * maxp, generator=g).to(torch.int32).reshape(len(lens), maxp)
    L = kf.layout("fp8t", Hkv, D, len(lens) * maxp)
    cache = torch.full((L.cache_bytes,), fill, dtype=torch.uint8, device="cuda")
    kept = {}
    for b, n in enumerate(lens):
        f = torch.exp(torch.empty(1, 1, D).uniform_(-1.5, 1.5, generator=g))
        k = (torch.randn(n, Hkv, D, generator=g) * f * 2).to(torch.bfloat16)
        tv = torch.exp(torch.empty(n, Hkv, 1).uniform_(-v_spread, v_spread, generator=g)) if v_spread else 1.0
        v = (torch.randn(n, Hkv, D, generator=g) * tv).to(torch.bfloat16)
        kept[b] = (k, v)
        if n:
            fk.quantize_append(L, k.cuda(), v.cuda(), wl.slots_for(table, b, 0, n).cuda(), cache)
    torch.cuda.synchronize()
    return L, cache, table, kept, g


def _reference(L, kept, lens, q, D):
    kv = [kf.stored_values("fp8t", L, kept[b][0]) for b in range(len(lens))]
    vv = [kf.stored_values("fp8t", L, kept[b][1]) for b in range(len(lens))]
    return oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, lens, D ** -0.5)


@pytest.mark.parametrize("G", [1, 3, 8, 16])
@pytest.mark.parametrize("splits", [0, 1, 5])
@pytest.mark.parametrize("D", [128, 64])
def test_decode_ragged_lengths(G, splits, D):
    """Lengths 0, 1, 31, 32, 33, 63, 64, 65, 1000: empty rows, both halves of
    a page ragged, NaN bytes in never-written slots."""
    lens = [0, 1, 31, 32, 33, 63, 64, 65, 1000]
    Hkv = 2
    L, cache, table, kept, g = _fill(lens, Hkv, D, seed=40 + G + D)
    q = torch.randn(len(lens), G * Hkv, D, generator=g).to(torch.bfloat16)
    _say(f"fp8 per-token decode: ragged lens {lens}, G={G}, splits={splits}, D={D}")
    out = fk.decode_attention(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda(),
                              num_splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = _reference(L, kept, lens, q, D)
    assert not out[0].any()
    err = float(hx.row_rel_error(out[1:], ref[1:]).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("spread", [3.0, 9.0])
@pytest.mark.parametrize("D", [128, 64])
def test_decode_v_scales_far_apart(spread, D):
    """V tokens whose magnitudes (and so scales) differ by up to e^(2 spread)
    within a page: the running V-scale reference moves up page by page and
    the weights p * s_v / R keep their precision."""
    lens = [70, 300, 2000]
    L, cache, table, kept, g = _fill(lens, 2, D, seed=int(spread) + D, v_spread=spread)
    q = torch.randn(len(lens), 8, D, generator=g).to(torch.bfloat16)
    _say(f"fp8 per-token decode: V magnitudes over e^+-{spread}, D={D}")
    out = fk.decode_attention(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda())
    torch.cuda.synchronize()
    err = float(hx.row_rel_error(out.cpu().numpy(), _reference(L, kept, lens, q, D)).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("name,seqs", [("gqa4_b8_ctx4k", None), ("gqa8_b32_ctx32k", [0, 31]),
                                       ("paged_b64_len1k_16k", [0, 17, 63])])
def test_decode_workloads(name, seqs):
    """Whole small workload, or sampled sequences of the 32K batch and the
    paged pool at their benchmark launch configuration; stored bytes of two
    checked sequences too."""
    w = wl.WORKLOADS[name]
    keep = range(w.batch) if seqs is None else seqs
    _say(f"fp8 per-token decode: {name}, checking sequences {list(keep)}")
    gc = hx.build_cache(w, seed=2, keep_seqs=keep, fmt="fp8t", zero=False)
    q = wl.queries(w, 2)
    out = fk.decode_attention(gc.layout, gc.cache, q.cuda(), gc.seq_lens, gc.page_table, num_splits=w.splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    lens = gc.lens_cpu.tolist()
    Hkv = w.kv_heads
    kv, vv = [], []
    for b in range(w.batch):
        if b in gc.kept:
            kv.append(kf.stored_values("fp8t", gc.layout, gc.kept[b][0]))
            vv.append(kf.stored_values("fp8t", gc.layout, gc.kept[b][1]))
        else:
            kv.append(np.zeros((1, Hkv, 128)))
            vv.append(np.zeros((1, Hkv, 128)))
    heads = [(b, h) for b in keep for h in range(Hkv)]
    ref = oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, lens, 128 ** -0.5, heads=heads)
    err = max(float(hx.row_rel_error(out[b], ref[b]).max()) for b in keep)
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL
    for b in list(keep)[:2]:
        n = lens[b]
        pages = gc.pt_cpu.table[b, : -(-n // 64)].tolist()
        k, v = gc.kept[b]
        kc, vc = hx.read_pages_fp8(gc.cache, gc.layout, pages, n)
        ksc, vsc = hx.read_token_scales(gc.cache, gc.layout, pages, n)
        ek, eks = oracle.quantize_fp8_groups(wl.bf16_bits(k), "token")
        ev, evs = oracle.quantize_fp8_groups(wl.bf16_bits(v), "token")
        assert np.array_equal(kc, ek) and np.array_equal(ksc, eks)
        assert np.array_equal(vc, ev) and np.array_equal(vsc, evs)
