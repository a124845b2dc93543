"""GPU tests of the decode step that stores its own token
(fp4kv_decode_append_attention): identical output and cache bytes to
quantize_append followed by decode_attention, for the fused kernels (FP4 at
D = 128, FP8) and the two-kernel path (FP4 at D = 64, the vector-ALU kernel),
and within 1e-3 per row of the oracle over the whole context."""

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


def _setup(lens, Hkv, G, D, fmt, seed, extra=1):
    """A cache holding lens[b] - 1 tokens per sequence (random page order,
    0x5A in never-written bytes), the new tokens, queries and page table."""
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    maxp = max(1, max(-(-(n + extra) // 64) for n in lens))
    table = torch.randperm(B * maxp, generator=g).to(torch.int32).reshape(B, maxp)
    L = kf.layout(fmt, Hkv, D, B * maxp)
    cache = torch.full((L.cache_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    kv = {}
    for b, n in enumerate(lens):
        k = (torch.randn(max(n, 0) + extra, Hkv, D, generator=g) * 2).to(torch.bfloat16)
        v = torch.randn(max(n, 0) + extra, Hkv, D, generator=g).to(torch.bfloat16)
        kv[b] = (k, v)
        if n > 1:
            fk.quantize_append(L, k[: n - 1].cuda(), v[: n - 1].cuda(), wl.slots_for(table, b, 0, n - 1).cuda(), cache)
    q = torch.randn(B, Hkv * G, D, generator=g).to(torch.bfloat16)
    torch.cuda.synchronize()
    return L, cache, table, kv, q


def _new_rows(kv, lens, Hkv, D, step=0):
    """bf16 [B][Hkv][D] of each sequence's token at position lens[b] - 1 + step
    (zeros for empty sequences)."""
    rows_k, rows_v = [], []
    for b, n in enumerate(lens):
        if n + step >= 1:
            rows_k.append(kv[b][0][n - 1 + step])
            rows_v.append(kv[b][1][n - 1 + step])
        else:
            rows_k.append(torch.zeros(Hkv, D, dtype=torch.bfloat16))
            rows_v.append(torch.zeros(Hkv, D, dtype=torch.bfloat16))
    return torch.stack(rows_k), torch.stack(rows_v)


def _unfused(L, cache, table, lens, kn, vn, q, splits, kernel="auto"):
    slots = []
    for b, n in enumerate(lens):
        slots.append(int(wl.slots_for(table, b, n - 1, n)[0]) if n >= 1 else -1)
    fk.quantize_append(L, kn.cuda(), vn.cuda(), torch.tensor(slots, dtype=torch.int64).cuda(), cache)
    return fk.decode_with_options(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda(),
                                  num_splits=splits, kernel=kernel)


CASES = [("fp4", 128, None), ("fp4", 64, None), ("fp8", 128, None), ("fp8", 64, None), ("fp8t", 128, None),
         ("fp8t", 64, None), ("fp4", 128, "valu")]
LENS = [0, 1, 2, 63, 64, 65, 128, 129, 1000, 4097]


@pytest.mark.parametrize("fmt,D,kernel", CASES)
@pytest.mark.parametrize("G,splits", [(1, 0), (4, 1), (8, 3), (16, 0), (3, 1000)])
def test_same_as_append_then_decode(fmt, D, kernel, G, splits):
    Hkv = 2
    L, cache, table, kv, q = _setup(LENS, Hkv, G, D, fmt, seed=G * 7 + D + splits)
    kn, vn = _new_rows(kv, LENS, Hkv, D)
    ref_cache = cache.clone()
    _say(f"append+decode: {fmt} D {D} kernel {kernel or 'default'} G {G} splits {splits}")
    lens_d = torch.tensor(LENS, dtype=torch.int32).cuda()
    if kernel:
        out = fk.decode_with_options(L, cache, q.cuda(), lens_d, table.cuda(), k_new=kn.cuda(), v_new=vn.cuda(),
                                     num_splits=splits, kernel=kernel)
        ref = _unfused(L, ref_cache, table, LENS, kn, vn, q, splits, kernel)
    else:
        out = fk.decode_append_attention(L, cache, kn.cuda(), vn.cuda(), q.cuda(), lens_d, table.cuda(),
                                         num_splits=splits)
        ref = _unfused(L, ref_cache, table, LENS, kn, vn, q, splits)
    torch.cuda.synchronize()
    assert torch.equal(cache, ref_cache)
    assert torch.equal(out, ref)


@pytest.mark.parametrize("fmt,D", [("fp4", 128), ("fp8", 128), ("fp4", 64), ("fp8", 64), ("fp8t", 128),
                                   ("fp8t", 64)])
def test_steps_against_oracle(fmt, D):
    """Five consecutive steps (positions of both parities, page crossings);
    the stored bytes and the last step's attention against the oracle."""
    lens0 = [1, 62, 63, 127, 300]
    Hkv, G = 2, 4
    L, cache, table, kv, q = _setup(lens0, Hkv, G, D, fmt, seed=11 + D, extra=5)
    for step in range(5):
        lens = [n + step for n in lens0]
        kn, vn = _new_rows(kv, lens0, Hkv, D, step)
        _say(f"append+decode step {step}: {fmt} D {D} lens {lens}")
        out = fk.decode_append_attention(L, cache, kn.cuda(), vn.cuda(), q.cuda(),
                                         torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda())
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    lens = [n + 4 for n in lens0]
    pages = [table[b, : -(-n // 64)].tolist() for b, n in enumerate(lens)]
    if fmt == "fp8t":
        for b, n in enumerate(lens):
            gk, gv = hx.read_pages_fp8(cache, L, pages[b], n)
            gks, gvs = hx.read_token_scales(cache, L, pages[b], n)
            ek, eks = oracle.quantize_fp8_groups(wl.bf16_bits(kv[b][0][:n]), "token")
            ev, evs = oracle.quantize_fp8_groups(wl.bf16_bits(kv[b][1][:n]), "token")
            assert np.array_equal(gk, ek) and np.array_equal(gks, eks)
            assert np.array_equal(gv, ev) and np.array_equal(gvs, evs)
        kvals = [kf.stored_values(fmt, L, kv[b][0][:n]) for b, n in enumerate(lens)]
        vvals = [kf.stored_values(fmt, L, kv[b][1][:n]) for b, n in enumerate(lens)]
        ref = oracle.decode_attention_values(wl.bf16_bits(q), kvals, vvals, lens, D ** -0.5)
    elif fmt == "fp8":
        ks, vs = L.params.k_scale, L.params.v_scale
        kc = [oracle.quantize_fp8(wl.bf16_bits(kv[b][0][:n]), ks) for b, n in enumerate(lens)]
        vc = [oracle.quantize_fp8(wl.bf16_bits(kv[b][1][:n]), vs) for b, n in enumerate(lens)]
        for b, n in enumerate(lens):
            gk, gv = hx.read_pages_fp8(cache, L, pages[b], n)
            assert np.array_equal(gk, kc[b]) and np.array_equal(gv, vc[b])
        ref = oracle.decode_attention_fp8(wl.bf16_bits(q), kc, vc, ks, vs, lens, D ** -0.5)
    else:
        kq = [oracle.quantize(wl.bf16_bits(kv[b][0][:n]), want_xhat=False) for b, n in enumerate(lens)]
        vq = [oracle.quantize(wl.bf16_bits(kv[b][1][:n]), want_xhat=False) for b, n in enumerate(lens)]
        for b, n in enumerate(lens):
            gkc, gks, gvc, gvs = hx.read_pages(cache, L, pages[b], n)
            assert np.array_equal(gkc, oracle.pack_nibbles(kq[b][0])) and np.array_equal(gks, kq[b][1])
            assert np.array_equal(gvc, oracle.pack_nibbles(vq[b][0])) and np.array_equal(gvs, vq[b][1])
        ref = oracle.decode_attention(wl.bf16_bits(q), [k[0] for k in kq], [k[1] for k in kq],
                                      [v[0] for v in vq], [v[1] for v in vq], lens, D ** -0.5)
    err = float(hx.row_rel_error(out, ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL


def test_skipped_page_and_empty_sequences():
    """A sequence whose last page id is out of range appends nothing and
    attends over its other pages (as decode_attention skips that page); a
    length of 0 appends nothing and gives a zero row."""
    lens = [0, 70, 130]
    Hkv, G, D = 1, 4, 128
    L, cache, table, kv, q = _setup(lens, Hkv, G, D, "fp4", seed=5)
    table = table.clone()
    table[1, 1] = L.num_pages + 3                       # page of position 69: out of range
    kn, vn = _new_rows(kv, lens, Hkv, D)
    before = cache.clone()
    out = fk.decode_append_attention(L, cache, kn.cuda(), vn.cuda(), q.cuda(),
                                     torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda())
    ref_cache = before.clone()
    slots = [-1, -1, int(wl.slots_for(table, 2, 129, 130)[0])]
    fk.quantize_append(L, kn.cuda(), vn.cuda(), torch.tensor(slots, dtype=torch.int64).cuda(), ref_cache)
    ref = fk.decode_attention(L, ref_cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda())
    torch.cuda.synchronize()
    assert torch.equal(cache, ref_cache)
    assert torch.equal(out, ref)
    assert not out[0].any()



@pytest.mark.parametrize("fmt,kernel", [("fp4", "auto"), ("fp4", "valu"), ("fp8", "auto")])
def test_dead_first_page_then_token_page(fmt, kernel):
    """The chunk's first page id is out of range and the token's page is the
    next one: the token's stores must land before that page is read.  One
    chunk covers both pages (one split), so the page loop starts at the dead
    page.  Bytes and output equal quantize_append + decode_attention."""
    lens = [100, 90, 128]                               # positions 99, 89, 127: page 1 of each
    Hkv, G, D = 2, 8, 128
    L, cache, table, kv, q = _setup(lens, Hkv, G, D, fmt, seed=17)
    table = table.clone()
    table[:, 0] = -1                                    # every sequence's first page is skipped
    kn, vn = _new_rows(kv, lens, Hkv, D)
    ref_cache = cache.clone()
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    _say(f"append+decode with a dead first page: {fmt} kernel {kernel}")
    out = fk.decode_with_options(L, cache, q.cuda(), lens_d, table.cuda(), k_new=kn.cuda(), v_new=vn.cuda(),
                                 num_splits=1, kernel=kernel)
    ref = _unfused(L, ref_cache, table, lens, kn, vn, q, 1, kernel)
    torch.cuda.synchronize()
    assert torch.equal(cache, ref_cache)
    assert torch.equal(out, ref)


@pytest.mark.parametrize("fmt,kernel", [("fp4", "auto"), ("fp4", "valu"), ("fp8", "auto"), ("fp8t", "auto")])
def test_length_past_the_table_appends_nothing(fmt, kernel):
    """seq_lens[b] above max_pages * 64: the token's position is not in the
    table, so nothing is stored (the last valid token is not overwritten);
    attention clamps the length, as decode_attention does."""
    lens = [128, 70]
    Hkv, G, D = 1, 4, 128
    L, cache, table, kv, q = _setup(lens, Hkv, G, D, fmt, seed=23, extra=0)
    assert table.shape[1] == 2                          # room for 128 tokens per sequence
    # sequence 0 holds 127 tokens; fill its last slot so that an overwrite would show
    fk.quantize_append(L, kv[0][0][127:128].cuda(), kv[0][1][127:128].cuda(),
                       wl.slots_for(table, 0, 127, 128).cuda(), cache)
    torch.cuda.synchronize()
    kn = torch.randn(2, Hkv, D).to(torch.bfloat16) * 5
    vn = torch.randn(2, Hkv, D).to(torch.bfloat16) * 5
    before = cache.clone()
    over = [129, 70]                                    # 129 > 2 * 64
    _say(f"append+decode with a length past the table: {fmt} kernel {kernel}")
    out = fk.decode_with_options(L, cache, q.cuda(), torch.tensor(over, dtype=torch.int32).cuda(), table.cuda(),
                                 k_new=kn.cuda(), v_new=vn.cuda(), kernel=kernel)
    ref_cache = before.clone()
    slots = [-1, int(wl.slots_for(table, 1, 69, 70)[0])]
    fk.quantize_append(L, kn.cuda(), vn.cuda(), torch.tensor(slots, dtype=torch.int64).cuda(), ref_cache)
    ref = fk.decode_with_options(L, ref_cache, q.cuda(), torch.tensor([128, 70], dtype=torch.int32).cuda(),
                                 table.cuda(), kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(cache, ref_cache)
    assert torch.equal(out, ref)
