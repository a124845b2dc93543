"""GPU parity of fp4kv_quantize_append: stored bytes bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_harness as hx
import fp4kv_workloads as wl
import oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _quantize_on_gpu(k, v, slots=None, num_pages=None):
    """Append bf16 [n][H][D] rows at `slots` (default 0..n-1) into a zeroed
    cache; returns (layout, device cache)."""
    n, H, D = k.shape
    if slots is None:
        slots = torch.arange(n, dtype=torch.int64)
    if num_pages is None:
        num_pages = max(1, -(-int(slots.max()) // 64) + 1) if n else 1
    layout = fk.cache_layout(H, D, num_pages)
    cache = torch.zeros(layout.cache_bytes, dtype=torch.uint8, device="cuda")
    fk.quantize_append(layout, k.cuda(), v.cuda(), slots.cuda(), cache)
    torch.cuda.synchronize()
    return layout, cache


def _expect(x):
    """Oracle codes of bf16 rows [n][H][D] as stored: packed code bytes and
    scale codes."""
    nib, sc, _ = oracle.quantize(wl.bf16_bits(x), want_xhat=False)
    return oracle.pack_nibbles(nib), sc


def _check_tokens(layout, cache, k, v, n):
    pages = list(range(-(-n // 64)))
    kc, ks, vc, vs = hx.read_pages(cache, layout, pages, n)
    ek, eks = _expect(k)
    ev, evs = _expect(v)
    assert np.array_equal(kc, ek)
    assert np.array_equal(ks, eks)
    assert np.array_equal(vc, ev)
    assert np.array_equal(vs, evs)


def _to_rows(blocks_u16, H=1, D=128):
    """[n_blocks][16] bf16 bits -> bf16 tensor [n_tokens][H][D] (zero padded)."""
    per = H * D // 16
    n_tok = -(-blocks_u16.shape[0] // per)
    pad = np.zeros((n_tok * per, 16), np.uint16)
    pad[: blocks_u16.shape[0]] = blocks_u16
    return torch.from_numpy(pad.view(np.int16).reshape(n_tok, H, D)).view(torch.bfloat16)


# token rows of 256 B to 2 KB: one KV head up to several per wave of the
# 16-token slice kernel, at D = 128 and 64
SHAPES = [(1, 128), (4, 128), (8, 128), (8, 64), (16, 64)]


@pytest.mark.parametrize("H,D", SHAPES)
def test_scale_rule_every_bf16_amax(H, D):
    """Blocks [a, 0, ..., 0] and [-a, ...] for every finite bf16 magnitude a
    (the maximum in either half of the block)."""
    a = np.arange(0, 0x7F80, dtype=np.uint16)
    blocks = np.zeros((2 * a.size, 16), np.uint16)
    blocks[0::2, 0] = a
    blocks[1::2, 13] = a | 0x8000
    k = _to_rows(blocks, H, D)
    v = _to_rows(blocks[::-1].copy(), H, D)
    _say(f"quantize_append: every bf16 amax, H {H} D {D}, {k.shape[0]} tokens")
    layout, cache = _quantize_on_gpu(k, v)
    _check_tokens(layout, cache, k, v, k.shape[0])


@pytest.mark.parametrize("H,D", SHAPES)
def test_element_rule_every_scale_and_magnitude(H, D):
    """For each of the 126 scale codes, every bf16 magnitude up to the largest
    block maximum that yields it, both signs, 15 per block behind that
    maximum."""
    a = np.arange(1, 0x7F80, dtype=np.uint16)
    _, sc, _ = oracle.quantize(a.reshape(-1, 1), want_xhat=False)
    best = {}
    for bits, code in zip(a, sc[:, 0]):
        best[int(code)] = int(bits)
    assert sorted(best) == list(range(1, 127))
    mags = np.arange(0, 0x7F80, dtype=np.uint16)
    chunks = []
    for code, amax in best.items():
        v = mags[mags <= amax]
        v = np.concatenate([v, v | 0x8000])
        nb = -(-v.size // 15)
        blk = np.zeros((nb, 16), np.uint16)
        blk[:, 0] = amax
        flat = np.zeros(nb * 15, np.uint16)
        flat[: v.size] = v
        blk[:, 1:] = flat.reshape(nb, 15)
        chunks.append(blk)
    blocks = np.concatenate(chunks)
    k = _to_rows(blocks, H, D)
    v = _to_rows(np.roll(blocks, 7, axis=0), H, D)
    _say(f"quantize_append: element rule, H {H} D {D}, {blocks.shape[0]} blocks, {k.shape[0]} tokens")
    layout, cache = _quantize_on_gpu(k, v)
    _check_tokens(layout, cache, k, v, k.shape[0])


@pytest.mark.parametrize("name", ["tiny_d64_ctx256", "gqa4_b8_ctx4k"])
def test_full_cache_small_workloads(name):
    w = wl.WORKLOADS[name]
    _say(f"quantize_append: full cache of {name}")
    gc = hx.build_cache(w, seed=1, keep_seqs=range(w.batch))
    for b in range(w.batch):
        k, v = gc.kept[b]
        n = int(gc.lens_cpu[b])
        kc, ks, vc, vs = hx.read_pages(gc.cache, gc.layout, gc.pt_cpu.table[b, : -(-n // 64)].tolist(), n)
        ek, eks = _expect(k)
        ev, evs = _expect(v)
        assert np.array_equal(kc, ek) and np.array_equal(ks, eks), f"K of sequence {b}"
        assert np.array_equal(vc, ev) and np.array_equal(vs, evs), f"V of sequence {b}"


@pytest.mark.parametrize("name,seqs", [("gqa8_b32_ctx32k", [0, 31]), ("gqa4_b1_ctx512k", [0]),
                                       ("paged_b64_len1k_16k", [0, 17, 63])])
def test_full_cache_large_workloads_sampled(name, seqs):
    """The whole cache is quantised as the benchmark does; the oracle checks
    sampled sequences (C3, C4) and the paged pool with its random page order."""
    w = wl.WORKLOADS[name]
    _say(f"quantize_append: full cache of {name}, checking sequences {seqs}")
    gc = hx.build_cache(w, seed=1, keep_seqs=seqs)
    for b in seqs:
        k, v = gc.kept[b]
        n = int(gc.lens_cpu[b])
        pages = gc.pt_cpu.table[b, : -(-n // 64)].tolist()
        kc, ks, vc, vs = hx.read_pages(gc.cache, gc.layout, pages, n)
        ek, eks = _expect(k)
        ev, evs = _expect(v)
        assert np.array_equal(kc, ek) and np.array_equal(ks, eks), f"K of sequence {b}"
        assert np.array_equal(vc, ev) and np.array_equal(vs, evs), f"V of sequence {b}"


def test_prefill_workload_full():
    w = wl.WORKLOADS["prefill_b8_8k"]
    _say("quantize_append: prefill 8 x 8192 tokens in one call")
    f_k, f_v = wl.channel_factors(w, 2, "k"), wl.channel_factors(w, 2, "v")
    k = torch.cat([wl.kv_tokens(w, 2, b, "k", 0, w.context, f_k) for b in range(w.batch)])
    v = torch.cat([wl.kv_tokens(w, 2, b, "v", 0, w.context, f_v) for b in range(w.batch)])
    layout, cache = _quantize_on_gpu(k, v)
    _check_tokens(layout, cache, k, v, k.shape[0])


def test_append_order_does_not_matter():
    """One call, token by token, and a shuffled order give identical bytes
    (a block never spans tokens)."""
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    k = wl.kv_tokens(w, 5, 0, "k", 0, 200)
    v = wl.kv_tokens(w, 5, 0, "v", 0, 200)
    _say("quantize_append: order invariance, 200 tokens")
    layout, ref = _quantize_on_gpu(k, v, num_pages=4)
    c1 = torch.zeros_like(ref)
    kd, vd = k.cuda(), v.cuda()
    for t in range(200):
        fk.quantize_append(layout, kd[t:t + 1], vd[t:t + 1], torch.tensor([t], device="cuda"), c1)
    perm = torch.randperm(200, generator=torch.Generator().manual_seed(0))
    c2 = torch.zeros_like(ref)
    fk.quantize_append(layout, kd[perm.cuda()].contiguous(), vd[perm.cuda()].contiguous(),
                       perm.cuda(), c2)
    torch.cuda.synchronize()
    assert torch.equal(ref, c1)
    assert torch.equal(ref, c2)


@pytest.mark.parametrize("first_slot,n", [(3, 1000), (8, 600), (0, 515), (64, 4096), (48, 530)])
def test_contiguous_runs_aligned_or_not(first_slot, n):
    """Long appends take 16-token slices: slices on 16-slot boundaries are
    written whole, misaligned or partial ones token by token; both give the
    oracle's bytes and leave the neighbouring slots untouched."""
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    k = wl.kv_tokens(w, 8, 0, "k", 0, n)
    v = wl.kv_tokens(w, 8, 0, "v", 0, n)
    pages = -(-(first_slot + n + 1) // 64)
    layout = fk.cache_layout(w.kv_heads, w.head_dim, pages)
    cache = torch.full((layout.cache_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    slots = torch.arange(first_slot, first_slot + n, dtype=torch.int64)
    _say(f"quantize_append: {n} tokens from slot {first_slot}")
    fk.quantize_append(layout, k.cuda(), v.cuda(), slots.cuda(), cache)
    torch.cuda.synchronize()
    kc, ks, vc, vs = hx.read_pages(cache, layout, list(range(pages)), pages * 64)
    ek, eks = _expect(k)
    ev, evs = _expect(v)
    sl = slice(first_slot, first_slot + n)
    assert np.array_equal(kc[sl], ek) and np.array_equal(ks[sl], eks)
    assert np.array_equal(vc[sl], ev) and np.array_equal(vs[sl], evs)
    # V bytes of untouched slots: each stored byte mixes two tokens, so check
    # the neighbours' nibbles through the token-major view
    for s in (first_slot - 1, first_slot + n):
        if 0 <= s < pages * 64:
            assert (vs[s] == 0x5A).all() and (ks[s] == 0x5A).all()
            nib = 0xA if s % 2 == 0 else 0x5          # even tokens sit in the low nibble
            assert (vc[s] == (nib | nib << 4)).all()


@pytest.mark.parametrize("H,D,first_slot,n", [(16, 128, 0, 1024), (16, 128, 5, 700), (32, 64, 16, 640),
                                              (2, 128, 0, 512), (16, 64, 32, 544)])
def test_slices_at_other_row_widths(H, D, first_slot, n):
    """The slice kernel where a wave's 64 blocks are part of a token row
    (H_kv 16 at D 128, H_kv 32 at D 64), exactly one row (H_kv 16 at D 64)
    or several tokens' rows (H_kv 2): the oracle's bytes at every slot,
    whole and misaligned slices alike."""
    g = torch.Generator().manual_seed(H * 1000 + D + first_slot)
    f = torch.exp(torch.empty(H, D).uniform_(-2.0, 2.0, generator=g))
    k = (torch.randn(n, H, D, generator=g) * f).to(torch.bfloat16)
    v = (torch.randn(n, H, D, generator=g) * f.flip(1)).to(torch.bfloat16)
    pages = -(-(first_slot + n) // 64)
    layout = fk.cache_layout(H, D, pages)
    cache = torch.zeros(layout.cache_bytes, dtype=torch.uint8, device="cuda")
    slots = torch.arange(first_slot, first_slot + n, dtype=torch.int64)
    _say(f"quantize_append: H_kv {H}, D {D}, {n} tokens from slot {first_slot}")
    fk.quantize_append(layout, k.cuda(), v.cuda(), slots.cuda(), cache)
    torch.cuda.synchronize()
    kc, ks, vc, vs = hx.read_pages(cache, layout, list(range(pages)), pages * 64)
    ek, eks = _expect(k)
    ev, evs = _expect(v)
    sl = slice(first_slot, first_slot + n)
    assert np.array_equal(kc[sl], ek) and np.array_equal(ks[sl], eks)
    assert np.array_equal(vc[sl], ev) and np.array_equal(vs[sl], evs)


def test_skipped_slots_leave_bytes_untouched():
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    k = wl.kv_tokens(w, 6, 0, "k", 0, 6)
    v = wl.kv_tokens(w, 6, 0, "v", 0, 6)
    layout = fk.cache_layout(w.kv_heads, w.head_dim, 2)
    cache = torch.full((layout.cache_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    slots = torch.tensor([3, -1, 127, 128, 1 << 40, 70], dtype=torch.int64)
    _say("quantize_append: negative and out-of-range slots")
    fk.quantize_append(layout, k.cuda(), v.cuda(), slots.cuda(), cache)
    torch.cuda.synchronize()
    kc, ks, vc, vs = hx.read_pages(cache, layout, [0, 1], 128)
    ek, eks = _expect(k)
    written = {3: 0, 127: 2, 70: 5}
    for s in range(128):
        if s in written:
            assert np.array_equal(kc[s], ek[written[s]]) and np.array_equal(ks[s], eks[written[s]])
        else:
            assert (kc[s] == 0xA5).all() and (vs[s] == 0xA5).all()
            nib = 0x5 if s % 2 == 0 else 0xA          # even tokens sit in the low nibble
            assert (vc[s] == (nib | nib << 4)).all()


def test_zero_tokens_is_a_no_op():
    layout = fk.cache_layout(2, 64, 1)
    cache = torch.zeros(layout.cache_bytes, dtype=torch.uint8, device="cuda")
    e = torch.empty(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    fk.quantize_append(layout, e, e, torch.empty(0, dtype=torch.int64, device="cuda"), cache)
    torch.cuda.synchronize()
    assert int(cache.sum()) == 0
