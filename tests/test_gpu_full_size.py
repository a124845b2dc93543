"""Parity at the full sizes the benchmark times, in its launch configurations.

- the 32-sequence, 32K-context batch at 64 chunks: every sequence, through
  fp4kv_decode_attention and through fp4kv_decode_with_options given the
  batch's shortest length (the chunk cut of uniform batches);
- the 512K-token sequence at 256 chunks: every KV head;
- the paged 64-sequence batch (lengths 1024..16384, random page table,
  automatic split count): three consecutive steps through
  fp4kv_decode_append_attention, each appending one token per sequence from
  inside the split kernel, and the last step again through the options call
  given the shortest length, as the benchmark makes it (same bits).  Every appended slot's bytes must equal the
  oracle's codes of that token; after the first step 8 sequences (the
  shortest and the longest among them), after the last step all 64, must be
  within 1e-3 per row of the oracle's attention.

The oracle quantises the same bf16 rows itself and attends in fp64; it runs
a few sequences at a time so that host memory stays bounded.
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
SEED = 1


def _say(msg):
    print(msg, flush=True)


def _codes(rows):
    nib, sc, _ = oracle.quantize(wl.bf16_bits(rows), want_xhat=False)
    return nib, sc


def _oracle_rows(w, q, rows_of, lens, seqs):
    """fp64 attention of the given sequences; rows_of(b) -> (k, v) bf16 rows."""
    H, D = w.kv_heads, w.head_dim
    empty = (np.zeros((0, H, D), np.uint8), np.zeros((0, H, D // 16), np.uint8))
    kc, ks, vc, vs = [], [], [], []
    for b in range(w.batch):
        if b in seqs:
            k, v = rows_of(b)
            (a, sa), (c, sc) = _codes(k), _codes(v)
        else:
            (a, sa), (c, sc) = empty, empty
        kc.append(a); ks.append(sa); vc.append(c); vs.append(sc)
    heads = [(b, h) for b in seqs for h in range(H)]
    return oracle.decode_attention(wl.bf16_bits(q), kc, ks, vc, vs, lens, D ** -0.5, heads=heads)


def test_gqa8_ctx32k_every_sequence():
    w = wl.WORKLOADS["gqa8_b32_ctx32k"]
    _say(f"full size: {w.name}, {w.splits} splits, all {w.batch} sequences")
    gc = hx.build_cache(w, seed=SEED)
    q = wl.queries(w, SEED)
    maxp = gc.page_table.shape[1]
    cut = fk.decode_chunks(gc.layout, w.batch, w.q_heads, maxp, w.splits, min_seq_len=w.context)
    _say(f"  chunks with the shortest length given: {tuple(cut)}")
    assert cut.tail_pages < cut.lead_pages and cut != fk.decode_chunks(gc.layout, w.batch, w.q_heads, maxp, w.splits)
    outs = {}
    outs["plain"] = fk.decode_attention(gc.layout, gc.cache, q.cuda(), gc.seq_lens, gc.page_table,
                                        num_splits=w.splits)
    outs["hinted"] = fk.decode_with_options(gc.layout, gc.cache, q.cuda(), gc.seq_lens, gc.page_table,
                                            num_splits=w.splits, min_seq_len=w.context)
    torch.cuda.synchronize()
    outs = {k: o.cpu().numpy() for k, o in outs.items()}
    for o in outs.values():
        assert np.isfinite(o).all()
    del gc
    torch.cuda.empty_cache()
    fk_, fv_ = wl.channel_factors(w, SEED, "k"), wl.channel_factors(w, SEED, "v")
    lens = [w.context] * w.batch
    rows_of = lambda b: (wl.kv_tokens(w, SEED, b, "k", 0, w.context, fk_),
                         wl.kv_tokens(w, SEED, b, "v", 0, w.context, fv_))
    worst = {k: 0.0 for k in outs}
    for b0 in range(0, w.batch, 4):
        seqs = list(range(b0, b0 + 4))
        ref = _oracle_rows(w, q, rows_of, lens, seqs)
        for k, o in outs.items():
            worst[k] = max(worst[k], float(hx.row_rel_error(o[seqs], ref[seqs]).max()))
        _say(f"  sequences {seqs[0]}..{seqs[-1]}: worst per-row relative error so far " +
             ", ".join(f"{k} {e:.3e}" for k, e in worst.items()))
    assert max(worst.values()) <= TOL


def test_ctx512k_every_kv_head():
    w = wl.WORKLOADS["gqa4_b1_ctx512k"]
    _say(f"full size: {w.name}, {w.splits} splits, all {w.kv_heads} KV heads")
    gc = hx.build_cache(w, seed=SEED)
    q = wl.queries(w, SEED)
    out = fk.decode_attention(gc.layout, gc.cache, q.cuda(), gc.seq_lens, gc.page_table, num_splits=w.splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    del gc
    torch.cuda.empty_cache()
    fk_, fv_ = wl.channel_factors(w, SEED, "k"), wl.channel_factors(w, SEED, "v")
    k = wl.kv_tokens(w, SEED, 0, "k", 0, w.context, fk_)
    v = wl.kv_tokens(w, SEED, 0, "v", 0, w.context, fv_)
    _say("  oracle: quantising 524288 tokens, then fp64 attention for 8 KV heads")
    ref = _oracle_rows(w, q, lambda b: (k, v), [w.context], [0])
    errs = hx.row_rel_error(out[0], ref[0])                   # one per query head
    for h in range(w.kv_heads):
        _say(f"  KV head {h}: worst per-row relative error {float(errs[h * w.group:(h + 1) * w.group].max()):.3e}")
    assert float(errs.max()) <= TOL


def test_paged_fused_steps_at_full_size():
    w = wl.WORKLOADS["paged_b64_len1k_16k"]
    steps = 3
    B, H, D = w.batch, w.kv_heads, w.head_dim
    _say(f"full size: {w.name}, {steps} steps of fp4kv_decode_append_attention, automatic splits")
    gc = hx.build_cache(w, seed=SEED, extra_tokens=steps)
    L = gc.layout
    lens0 = [int(n) for n in gc.lens_cpu]
    table = gc.pt_cpu.table
    splits, partials, ws_bytes = fk.decode_plan(L, B, w.q_heads, table.shape[1], 0)
    _say(f"  lengths {min(lens0)}..{max(lens0)}, {L.num_pages} pages, plan: {splits} chunks, {partials} partials")
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    news, outs, qs = [], [], []
    for s in range(steps):
        kn, vn = wl.new_tokens(w, SEED, s)
        q = wl.queries(w, SEED, step=s)
        lens = torch.tensor([n + s + 1 for n in lens0], dtype=torch.int32)
        out = fk.decode_append_attention(L, gc.cache, kn.cuda(), vn.cuda(), q.cuda(), lens.cuda(), gc.page_table,
                                         workspace=ws)
        torch.cuda.synchronize()
        news.append((kn, vn))
        outs.append(out.cpu().numpy())
        qs.append(q)
        # the appended slots against the oracle's codes of the step's tokens
        pos = [n + s for n in lens0]
        pages = [int(table[b, p // 64]) for b, p in enumerate(pos)]
        gkc, gks, gvc, gvs = hx.read_pages(gc.cache, L, pages, 64 * B)
        rows = [64 * b + p % 64 for b, p in enumerate(pos)]
        (kc, ks), (vc, vs) = _codes(kn), _codes(vn)
        assert np.array_equal(gkc[rows], oracle.pack_nibbles(kc)) and np.array_equal(gks[rows], ks), s
        assert np.array_equal(gvc[rows], oracle.pack_nibbles(vc)) and np.array_equal(gvs[rows], vs), s
        _say(f"  step {s}: the {B} appended slots (K and V codes and scales) equal the oracle's")
    # the last step again as the benchmark makes it: the options call given the
    # shortest length (the same chunks here, so the same bits), appending the
    # same token again (the same bytes)
    cache_before = gc.cache.clone()
    kn, vn = news[-1]
    again = fk.decode_with_options(L, gc.cache, qs[-1].cuda(), lens.cuda(), gc.page_table, k_new=kn.cuda(),
                                   v_new=vn.cuda(), workspace=ws, min_seq_len=int(lens.min()))
    torch.cuda.synchronize()
    assert fk.decode_chunks(L, B, w.q_heads, table.shape[1], 0, min_seq_len=int(lens.min())) == \
        fk.decode_chunks(L, B, w.q_heads, table.shape[1], 0)
    assert torch.equal(gc.cache, cache_before)
    assert np.array_equal(again.cpu().numpy(), outs[-1])
    del cache_before
    _say("  the last step through the options call with the shortest length: the same cache bytes and output bits")

    factors = wl.channel_factors(w, SEED, "k"), wl.channel_factors(w, SEED, "v")

    def rows_of(b, n_new):
        k = wl.kv_tokens(w, SEED, b, "k", 0, lens0[b], factors[0])
        v = wl.kv_tokens(w, SEED, b, "v", 0, lens0[b], factors[1])
        k = torch.cat([k] + [news[s][0][b:b + 1] for s in range(n_new)])
        v = torch.cat([v] + [news[s][1][b:b + 1] for s in range(n_new)])
        return k, v

    order = sorted(range(B), key=lambda b: lens0[b])
    first = sorted({order[int(i)] for i in np.linspace(0, B - 1, 8).round()})   # shortest .. longest
    lens = [n + 1 for n in lens0]
    ref = _oracle_rows(w, qs[0], lambda b: rows_of(b, 1), lens, first)
    err = float(hx.row_rel_error(outs[0][first], ref[first]).max())
    _say(f"  step 0, sequences {first} (lengths {[lens[b] for b in first]}): worst per-row error {err:.3e}")
    assert len(first) >= 8 and err <= TOL
    lens = [n + steps for n in lens0]
    worst = 0.0
    for g0 in range(0, B, 8):
        seqs = list(range(g0, g0 + 8))
        ref = _oracle_rows(w, qs[-1], lambda b: rows_of(b, steps), lens, seqs)
        err = float(hx.row_rel_error(outs[-1][seqs], ref[seqs]).max())
        worst = max(worst, err)
        _say(f"  step {steps - 1}, sequences {g0}..{g0 + 7}: worst per-row relative error {err:.3e}")
    assert worst <= TOL
