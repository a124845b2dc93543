"""GPU parity of fp4kv_decode_attention against the fp64 oracle.

The oracle quantises the same bf16 rows itself and attends in fp64; the GPU
result must be within 1e-3 of it, measured per output row as
max |out - ref| / max |ref|.  fp32 accumulation over at most 2^19 tokens of
values that are exact in fp32 keeps the error orders of magnitude below that.
"""
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


def _oracle_codes(rows):
    nib, sc, _ = oracle.quantize(wl.bf16_bits(rows), want_xhat=False)
    return nib, sc


def _oracle_decode(q, kv_rows, lens, D, scale, heads=None):
    """kv_rows: dict seq -> (k, v) bf16 rows; sequences not in it are left 0."""
    B = q.shape[0]
    H = next(iter(kv_rows.values()))[0].shape[1]
    empty = np.zeros((0, H, D), np.uint8), np.zeros((0, H, D // 16), np.uint8)
    kc, ks, vc, vs = [], [], [], []
    for b in range(B):
        if b in kv_rows:
            a, sa = _oracle_codes(kv_rows[b][0][: lens[b]])
            c, sc = _oracle_codes(kv_rows[b][1][: lens[b]])
        else:
            a, sa = empty
            c, sc = empty
        kc.append(a); ks.append(sa); vc.append(c); vs.append(sc)
    if heads is None:
        heads = [(b, h) for b in kv_rows for h in range(H)]
    return oracle.decode_attention(wl.bf16_bits(q), kc, ks, vc, vs, lens, scale, heads=heads)


def _gpu_decode(gc, q, splits, scale=None):
    out = fk.decode_attention(gc.layout, gc.cache, q.cuda(), gc.seq_lens, gc.page_table,
                              softmax_scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _assert_close(out, ref, rows):
    """rows: list of (b, q-head range) to compare."""
    worst = 0.0
    for b, hs in rows:
        err = hx.row_rel_error(out[b, hs], ref[b, hs])
        worst = max(worst, float(err.max()))
    _say(f"  worst per-row relative error {worst:.3e}")
    assert worst <= TOL


@pytest.mark.parametrize("name,splits", [("tiny_d64_ctx256", 0), ("tiny_d64_ctx256", 1),
                                         ("gqa4_b8_ctx4k", 0), ("gqa4_b8_ctx4k", 7)])
def test_small_workloads_every_row(name, splits):
    w = wl.WORKLOADS[name]
    _say(f"decode_attention: {name}, splits={splits}")
    gc = hx.build_cache(w, seed=1, keep_seqs=range(w.batch))
    q = wl.queries(w, 1)
    out = _gpu_decode(gc, q, splits)
    lens = gc.lens_cpu.tolist()
    ref = _oracle_decode(q, gc.kept, lens, w.head_dim, w.head_dim ** -0.5)
    _assert_close(out, ref, [(b, slice(None)) for b in range(w.batch)])


def test_gqa8_ctx32k_sampled_sequences():
    w = wl.WORKLOADS["gqa8_b32_ctx32k"]
    seqs = [0, 31]
    _say(f"decode_attention: {w.name}, {w.splits} splits, oracle on sequences {seqs}")
    gc = hx.build_cache(w, seed=1, keep_seqs=seqs)
    q = wl.queries(w, 1)
    out = _gpu_decode(gc, q, w.splits)
    lens = gc.lens_cpu.tolist()
    ref = _oracle_decode(q, gc.kept, lens, w.head_dim, w.head_dim ** -0.5)
    _assert_close(out, ref, [(b, slice(None)) for b in seqs])
    assert np.isfinite(out).all()


def test_ctx512k_sampled_heads():
    w = wl.WORKLOADS["gqa4_b1_ctx512k"]
    heads = [(0, 0), (0, 5)]
    _say(f"decode_attention: {w.name}, {w.splits} splits, oracle on KV heads {heads}")
    gc = hx.build_cache(w, seed=1, keep_seqs=[0])
    q = wl.queries(w, 1)
    out = _gpu_decode(gc, q, w.splits)
    ref = _oracle_decode(q, gc.kept, gc.lens_cpu.tolist(), w.head_dim, w.head_dim ** -0.5, heads=heads)
    G = w.group
    _assert_close(out, ref, [(0, slice(h * G, (h + 1) * G)) for _, h in heads])


def test_paged_append_then_decode_step():
    """One step of the paged workload: every sequence appends one token at
    position len_b through its random page table, then attends over len_b + 1."""
    w = wl.WORKLOADS["paged_b64_len1k_16k"]
    seqs = [0, 17, 63]
    _say(f"decode_attention: {w.name}, append + attend, oracle on sequences {seqs}")
    gc = hx.build_cache(w, seed=1, keep_seqs=seqs, extra_tokens=1)
    knew, vnew = wl.new_tokens(w, 1, 0)
    slots = torch.stack([wl.slots_for(gc.pt_cpu.table, b, int(gc.lens_cpu[b]), int(gc.lens_cpu[b]) + 1)[0]
                         for b in range(w.batch)])
    fk.quantize_append(gc.layout, knew.cuda(), vnew.cuda(), slots.cuda(), gc.cache)
    gc.seq_lens += 1
    q = wl.queries(w, 1, step=0)
    out = _gpu_decode(gc, q, 0)
    kept = {b: (torch.cat([gc.kept[b][0], knew[b:b + 1]]), torch.cat([gc.kept[b][1], vnew[b:b + 1]]))
            for b in seqs}
    lens = (gc.lens_cpu + 1).tolist()
    ref = _oracle_decode(q, kept, lens, w.head_dim, w.head_dim ** -0.5)
    _assert_close(out, ref, [(b, slice(None)) for b in seqs])


def _custom_cache(B, Hq, Hkv, D, lens, seed, page_order="identity", kscale=1.0):
    """A small batch with the given lengths; returns (gc-like tuple pieces)."""
    g = torch.Generator().manual_seed(seed)
    maxp = max(1, max(-(-l // 64) for l in lens))
    if page_order == "identity":
        table = torch.arange(B * maxp, dtype=torch.int32).reshape(B, maxp)
    else:
        table = torch.randperm(B * maxp, generator=g).to(torch.int32).reshape(B, maxp)
    layout = fk.cache_layout(Hkv, D, B * maxp)
    cache = torch.zeros(layout.cache_bytes, dtype=torch.uint8, device="cuda")
    kept = {}
    for b, L in enumerate(lens):
        k = (torch.randn(L, Hkv, D, generator=g) * kscale).to(torch.bfloat16)
        v = torch.randn(L, Hkv, D, generator=g).to(torch.bfloat16)
        kept[b] = (k, v)
        if L:
            fk.quantize_append(layout, k.cuda(), v.cuda(), wl.slots_for(table, b, 0, L).cuda(), cache)
    q = torch.randn(B, Hq, D, generator=g).to(torch.bfloat16)
    return layout, cache, table, kept, q


@pytest.mark.parametrize("G,D", [(1, 128), (2, 64), (3, 128), (16, 128), (8, 64)])
@pytest.mark.parametrize("splits", [0, 1, 3, 1000])
def test_ragged_lengths_group_sizes_and_splits(G, D, splits):
    """Lengths 0, 1, 63, 64, 65 and 1000 in one batch (empty rows, ragged last
    pages, splits with no tokens), every supported group shape, random page
    order."""
    lens = [0, 1, 63, 64, 65, 1000]
    Hkv = 2
    _say(f"decode_attention: ragged lens {lens}, G={G}, D={D}, splits={splits}")
    layout, cache, table, kept, q = _custom_cache(len(lens), G * Hkv, Hkv, D, lens, 100 + G + D,
                                                  page_order="random", kscale=3.0)
    out = fk.decode_attention(layout, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                              table.cuda(), num_splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = _oracle_decode(q, kept, lens, D, D ** -0.5)
    assert np.array_equal(out[0], np.zeros_like(out[0]))          # empty context -> zeros
    _assert_close(out, ref, [(b, slice(None)) for b in range(1, len(lens))])


def test_invalid_page_ids_are_skipped():
    lens = [200]
    layout, cache, table, kept, q = _custom_cache(1, 4, 1, 128, lens, 7)
    table[0, 1] = -5                      # tokens 64..127 are not attended
    _say("decode_attention: a page id outside the pool")
    out = fk.decode_attention(layout, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                              table.cuda())
    torch.cuda.synchronize()
    keep = torch.cat([torch.arange(0, 64), torch.arange(128, 200)])
    k, v = kept[0]
    ref = _oracle_decode(q, {0: (k[keep], v[keep])}, [len(keep)], 128, 128 ** -0.5)
    _assert_close(out.cpu().numpy(), ref, [(0, slice(None))])


def test_deterministic_and_split_invariant():
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    gc = hx.build_cache(w, seed=3)
    q = wl.queries(w, 3)
    _say("decode_attention: repeat runs and split counts 1, 8, 64")
    a = _gpu_decode(gc, q, 8)
    b = _gpu_decode(gc, q, 8)
    assert np.array_equal(a, b)
    for s in (1, 64):
        c = _gpu_decode(gc, q, s)
        assert float(hx.row_rel_error(c, a.astype(np.float64)).max()) < 1e-4


def test_softmax_scale_argument():
    lens = [300]
    layout, cache, table, kept, q = _custom_cache(1, 8, 2, 128, lens, 9)
    _say("decode_attention: softmax_scale 0.3")
    out = fk.decode_attention(layout, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                              table.cuda(), softmax_scale=0.3)
    torch.cuda.synchronize()
    ref = _oracle_decode(q, kept, lens, 128, 0.3)
    _assert_close(out.cpu().numpy(), ref, [(0, slice(None))])


def test_workspace_reused_across_calls_and_shapes():
    """One workspace, filled with garbage first, serves consecutive calls of
    different batch sizes and split counts: every result equals the result
    with a fresh workspace."""
    lens = [0, 1, 63, 64, 65, 1000, 3000, 129]
    Hkv, G, D = 2, 4, 128
    layout, cache, table, kept, q = _custom_cache(len(lens), G * Hkv, Hkv, D, lens, 21, page_order="random")
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    q_d, table_d = q.cuda(), table.cuda()
    cases = [(8, 0), (3, 7), (8, 1), (5, 64), (8, 0)]
    plans = {c: fk.decode_plan(layout, c[0], G * Hkv, table.shape[1], c[1]) for c in cases}
    ws = torch.full((max(p.workspace_bytes for p in plans.values()),), 0xC3, dtype=torch.uint8, device="cuda")
    _say(f"decode_attention: one workspace for (batch, splits) = {cases}")
    for B, s in cases:
        out = fk.decode_attention(layout, cache, q_d[:B].contiguous(), lens_d[:B].contiguous(),
                                  table_d[:B].contiguous(), num_splits=s, workspace=ws)
        fresh = fk.decode_attention(layout, cache, q_d[:B].contiguous(), lens_d[:B].contiguous(),
                                    table_d[:B].contiguous(), num_splits=s)
        torch.cuda.synchronize()
        assert torch.equal(out, fresh), (B, s)
    ref = _oracle_decode(q, kept, lens, D, D ** -0.5)
    _assert_close(out.cpu().numpy(), ref, [(b, slice(None)) for b in range(1, len(lens))])
