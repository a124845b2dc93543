"""GPU parity of the decode kernels where the plan cuts the context into
lead and tail chunks of different sizes (fp4kv_decode_chunks: grids of at
least 1536 workgroups).  Sequence lengths sit on every chunk boundary (one
token before, at and after it), so that each way a chunk can end -- inside
a lead chunk, at the lead/tail seam, inside a tail chunk, at the table's
end -- occurs; every split kernel and cache format, the step that appends
its own token, and a sliding window with two query tokens are checked
against the oracle (1e-3 per output row) or, for the appended step,
against quantize_append followed by decode_attention (bit for bit).  The
cut for uniform batches (a shortest length given through
fp4kv_decode_with_options) is checked the same way, and so is a shortest
length the batch does not keep (the results must not depend on it)."""
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
HKV, G, D = 8, 4, 128
MAXP, SPLITS, BATCH = 48, 16, 64          # 8 x 64 x 4 = 2048 workgroups


def _say(msg):
    print(msg, flush=True)


def _boundary_lengths(chunks, n_chunks, maxp, batch, seed):
    """Lengths one token before, at and after every chunk start, 0, 1 and
    the table's end; seeded fill up to `batch`."""
    cuts = sorted({chunks.first_page(k) for k in range(1, n_chunks)} | {maxp})
    lens = {0, 1, maxp * 64}
    for c in cuts:
        lens |= {c * 64 - 1, c * 64, c * 64 + 1}
    lens = sorted(x for x in lens if 0 <= x <= maxp * 64)
    assert len(lens) <= batch, len(lens)
    rng = np.random.default_rng(seed)
    lens += [int(x) for x in rng.integers(0, maxp * 64 + 1, batch - len(lens))]
    rng.shuffle(lens)
    return lens


def _setup(lens, fmt, seed, maxp, extra=0):
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    table = torch.randperm(B * maxp, generator=g).to(torch.int32).reshape(B, maxp)
    L = kf.layout(fmt, HKV, D, B * maxp)
    cache = torch.full((L.cache_bytes,), 0x5A, dtype=torch.uint8, device="cuda")
    kv = {}
    for b, n in enumerate(lens):
        k = (torch.randn(n + extra, HKV, D, generator=g) * 2).to(torch.bfloat16)
        v = torch.randn(n + extra, HKV, D, generator=g).to(torch.bfloat16)
        kv[b] = (k, v)
        if n > 0:
            fk.quantize_append(L, k[:n].cuda(), v[:n].cuda(), wl.slots_for(table, b, 0, n).cuda(), cache)
    torch.cuda.synchronize()
    return L, cache, table, kv, g


def _oracle(fmt, L, kv, lens, q):
    """fp64 attention of q [B][Hq][D] over each sequence's first lens[b] tokens."""
    if fmt == "fp8t":
        kvals = [kf.stored_values(fmt, L, kv[b][0][:n]) if n else np.zeros((1, HKV, D)) for b, n in enumerate(lens)]
        vvals = [kf.stored_values(fmt, L, kv[b][1][:n]) if n else np.zeros((1, HKV, D)) for b, n in enumerate(lens)]
        return oracle.decode_attention_values(wl.bf16_bits(q), kvals, vvals, lens, D ** -0.5)
    if fmt == "fp8":
        ks, vs = L.params.k_scale, L.params.v_scale
        kc = [oracle.quantize_fp8(wl.bf16_bits(kv[b][0][:n]), ks) for b, n in enumerate(lens)]
        vc = [oracle.quantize_fp8(wl.bf16_bits(kv[b][1][:n]), vs) for b, n in enumerate(lens)]
        return oracle.decode_attention_fp8(wl.bf16_bits(q), kc, vc, ks, vs, lens, D ** -0.5)
    kq = [oracle.quantize(wl.bf16_bits(kv[b][0][:n]), want_xhat=False) for b, n in enumerate(lens)]
    vq = [oracle.quantize(wl.bf16_bits(kv[b][1][:n]), want_xhat=False) for b, n in enumerate(lens)]
    return oracle.decode_attention(wl.bf16_bits(q), [k[0] for k in kq], [k[1] for k in kq],
                                   [v[0] for v in vq], [v[1] for v in vq], lens, D ** -0.5)


def _chunks(fmt, batch=BATCH, maxp=MAXP, splits=SPLITS):
    L = kf.layout(fmt, HKV, D, 64)
    return fk.decode_plan(L, batch, HKV * G, maxp, splits), fk.decode_chunks(L, batch, HKV * G, maxp, splits)


def fk_span(maxp, q_tokens, window):
    """Pages a windowed plan covers (as the library documents it)."""
    return min(maxp, -(-(window + q_tokens - 1) // 64) + 1)


def test_plan_has_lead_and_tail_chunks():
    plan, ch = _chunks("fp4")
    _say(f"plan {tuple(plan)}, chunks {tuple(ch)}")
    assert plan.partials * HKV * BATCH >= 1536
    assert ch.tail_pages < ch.lead_pages and ch.lead_chunks < 4 * plan.partials
    assert ch.first_page(4 * plan.partials) >= MAXP              # the chunks cover the table


@pytest.mark.parametrize("fmt,kernel", [("fp4", "auto"), ("fp4", "mfma_direct"), ("fp4", "valu"), ("fp8", "auto"),
                                        ("fp8t", "auto")])
def test_boundary_lengths_against_oracle(fmt, kernel):
    plan, ch = _chunks(fmt)
    lens = _boundary_lengths(ch, 4 * plan.partials, MAXP, BATCH, seed=3)
    _say(f"lead/tail chunks {tuple(ch)}: {fmt} kernel {kernel}, lengths {sorted(lens)[:12]}..")
    L, cache, table, kv, g = _setup(lens, fmt, seed=5, maxp=MAXP)
    q = torch.randn(BATCH, HKV * G, D, generator=g).to(torch.bfloat16)
    out = fk.decode_with_options(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda(),
                                 num_splits=SPLITS, kernel=kernel)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = _oracle(fmt, L, kv, lens, q)
    err = float(hx.row_rel_error(out, ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert np.isfinite(out).all() and err <= TOL
    assert not out[[b for b, n in enumerate(lens) if n == 0]].any()


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_fused_append_equals_append_then_decode(fmt):
    plan, ch = _chunks(fmt)
    lens = _boundary_lengths(ch, 4 * plan.partials, MAXP, BATCH, seed=7)
    lens = [max(n, 1) for n in lens]                               # each sequence appends its token
    L, cache, table, kv, g = _setup([n - 1 for n in lens], fmt, seed=9, maxp=MAXP, extra=1)
    q = torch.randn(BATCH, HKV * G, D, generator=g).to(torch.bfloat16)
    kn = torch.stack([kv[b][0][n - 1] for b, n in enumerate(lens)])
    vn = torch.stack([kv[b][1][n - 1] for b, n in enumerate(lens)])
    ref_cache = cache.clone()
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    _say(f"fused append under lead/tail chunks {tuple(ch)}: {fmt}")
    out = fk.decode_append_attention(L, cache, kn.cuda(), vn.cuda(), q.cuda(), lens_d, table.cuda(),
                                     num_splits=SPLITS)
    slots = torch.tensor([int(wl.slots_for(table, b, n - 1, n)[0]) for b, n in enumerate(lens)], dtype=torch.int64)
    fk.quantize_append(L, kn.cuda(), vn.cuda(), slots.cuda(), ref_cache)
    ref = fk.decode_attention(L, ref_cache, q.cuda(), lens_d, table.cuda(), num_splits=SPLITS)
    torch.cuda.synchronize()
    assert torch.equal(cache, ref_cache)
    assert torch.equal(out, ref)


def test_window_two_query_tokens_against_oracle():
    """96 sequences, window 700, two query tokens: 2 partials per row over the
    window's span, whose chunks the plan cuts into lead and tail sizes."""
    B, window, S, maxp, splits = 96, 700, 2, 32, 7
    L0 = kf.layout("fp4", HKV, D, 64)
    ch = fk.decode_chunks(L0, B, HKV * G, maxp, splits, q_tokens=S, window=window)
    plan = fk.decode_window_plan(L0, B, S, HKV * G, maxp, window, splits)
    assert ch.tail_pages < ch.lead_pages, tuple(ch)
    span = fk_span(maxp, S, window)
    cuts = sorted({ch.first_page(k) for k in range(1, 4 * plan.partials)} | {span})
    # lengths whose window starts on either side of a page edge, so that the
    # window's chunks start at shifted pages too, plus short and full ones
    lens = sorted({0, 1, 2, 63, 64, 65, 700, 701, 702, maxp * 64} |
                  {c * 64 + d for c in cuts for d in (-1, 0, 1)} |
                  {c * 64 + 700 + d for c in (3, 7, 11) for d in (-1, 0, 1)})
    lens = [n for n in lens if 0 <= n <= maxp * 64]
    rng = np.random.default_rng(11)
    lens += [int(x) for x in rng.integers(0, maxp * 64 + 1, B - len(lens))]
    L, cache, table, kv, g = _setup(lens, "fp4", seed=13, maxp=maxp)
    q = torch.randn(B, S, HKV * G, D, generator=g).to(torch.bfloat16)
    _say(f"window {window}, {S} query tokens, chunks {tuple(ch)}, plan {tuple(plan)}")
    out = fk.decode_window_attention(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                                     table.cuda(), window, num_splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for b, n in enumerate(lens):
        kq = oracle.quantize(wl.bf16_bits(kv[b][0][:n]), want_xhat=False) if n else None
        vq = oracle.quantize(wl.bf16_bits(kv[b][1][:n]), want_xhat=False) if n else None
        for i in range(S):
            end = n - (S - 1 - i)
            if end <= 0:
                assert not out[b, i].any()
                continue
            lo = max(0, end - window)
            r = oracle.decode_attention(wl.bf16_bits(q[b:b + 1, i].contiguous()), [kq[0][lo:end]], [kq[1][lo:end]],
                                        [vq[0][lo:end]], [vq[1][lo:end]], [end - lo], D ** -0.5)
            worst = max(worst, float(hx.row_rel_error(out[b, i][None], r).max()))
    _say(f"  worst per-row relative error {worst:.3e}")
    assert worst <= TOL


def _hinted_lengths(ch, n_chunks, maxp, batch, lo, seed):
    """Lengths one token before, at and after every chunk start at or past
    page `lo`, and the table's end; seeded fill in [lo * 64, maxp * 64]."""
    cuts = sorted({ch.first_page(k) for k in range(1, n_chunks)} | {maxp})
    lens = {lo * 64, lo * 64 + 1, maxp * 64}
    for c in cuts:
        lens |= {c * 64 - 1, c * 64, c * 64 + 1}
    lens = sorted(x for x in lens if lo * 64 <= x <= maxp * 64)
    assert len(lens) <= batch, len(lens)
    rng = np.random.default_rng(seed)
    lens += [int(x) for x in rng.integers(lo * 64, maxp * 64 + 1, batch - len(lens))]
    rng.shuffle(lens)
    return lens


@pytest.mark.parametrize("fmt,kernel", [("fp4", "auto"), ("fp4", "mfma_direct"), ("fp4", "valu"), ("fp8", "auto"),
                                        ("fp8t", "auto")])
def test_shortest_length_cut_against_oracle(fmt, kernel):
    """Every sequence at least 7/8 of the table: with the shortest length
    given, the partials after the lead ones (the first generation's worth
    for FP4, a quarter or that for FP8) take one-page chunks."""
    plan = _chunks(fmt)[0]
    L0 = kf.layout(fmt, HKV, D, 64)
    lo = -(-7 * MAXP // 8)
    ch = fk.decode_chunks(L0, BATCH, HKV * G, MAXP, SPLITS, min_seq_len=lo * 64)
    fill = -(-768 // (HKV * BATCH))
    lead_parts = fill if fmt == "fp4" else max(fill, plan.partials - 3 * plan.partials // 4)
    assert ch.tail_pages == 1 < ch.lead_pages and ch.lead_chunks == 4 * lead_parts
    lens = _hinted_lengths(ch, 4 * plan.partials, MAXP, BATCH, lo, seed=15)
    _say(f"shortest-length cut {tuple(ch)}: {fmt} kernel {kernel}, lengths {sorted(lens)[:8]}..")
    L, cache, table, kv, g = _setup(lens, fmt, seed=17, maxp=MAXP)
    q = torch.randn(BATCH, HKV * G, D, generator=g).to(torch.bfloat16)
    out = fk.decode_with_options(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), table.cuda(),
                                 num_splits=SPLITS, kernel=kernel, min_seq_len=min(lens))
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = _oracle(fmt, L, kv, lens, q)
    err = float(hx.row_rel_error(out, ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert np.isfinite(out).all() and err <= TOL


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_shortest_length_not_kept_is_still_correct(fmt):
    """A shortest length the batch does not keep (ragged lengths from 0,
    promised the whole table) changes only the cut: the rows still match the
    oracle, and the split kernel alone (merge none) followed by the combine
    gives the same bits as the whole call."""
    plan, ch = _chunks(fmt)
    lens = _boundary_lengths(ch, 4 * plan.partials, MAXP, BATCH, seed=19)
    L, cache, table, kv, g = _setup(lens, fmt, seed=21, maxp=MAXP)
    q = torch.randn(BATCH, HKV * G, D, generator=g).to(torch.bfloat16).cuda()
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    wrong = MAXP * 64
    _say(f"{fmt}: ragged lengths, shortest length given as {wrong}")
    out = fk.decode_with_options(L, cache, q, lens_d, table.cuda(), num_splits=SPLITS, min_seq_len=wrong)
    ws, p = fk.decode_with_options(L, cache, q, lens_d, table.cuda(), num_splits=SPLITS, min_seq_len=wrong,
                                   merge="none")
    again = fk.decode_combine(ws, BATCH, HKV * G, D, p.partials)
    torch.cuda.synchronize()
    assert torch.equal(out, again)
    out = out.cpu().numpy()
    ref = _oracle(fmt, L, kv, lens, q.cpu())
    err = float(hx.row_rel_error(out, ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert np.isfinite(out).all() and err <= TOL
    assert not out[[b for b, n in enumerate(lens) if n == 0]].any()


def test_window_with_shortest_length_against_oracle():
    """A 2,000-token window over 96 sequences whose plan differs when every
    sequence is promised the whole table (most are shorter): both cuts of the
    window's span, against the oracle's windowed attention."""
    B, window, maxp, splits = 96, 2000, 48, 16
    L0 = kf.layout("fp4", HKV, D, 64)
    plan = fk.decode_window_plan(L0, B, 1, HKV * G, maxp, window, splits)
    ch = fk.decode_chunks(L0, B, HKV * G, maxp, splits, window=window)
    ch_h = fk.decode_chunks(L0, B, HKV * G, maxp, splits, window=window, min_seq_len=maxp * 64)
    span = fk_span(maxp, 1, window)
    assert ch != ch_h and ch_h.tail_pages < ch_h.lead_pages, (tuple(ch), tuple(ch_h))
    cuts = sorted({c.first_page(k) for c in (ch, ch_h) for k in range(1, 4 * plan.partials)} | {span})
    lens = sorted({0, 1, 64, 1999, 2000, 2001, maxp * 64} |
                  {c * 64 + d for c in cuts for d in (-1, 0, 1)} |
                  {c * 64 + window + d for c in (1, 5, 9) for d in (-1, 0, 1)})
    lens = [n for n in lens if 0 <= n <= maxp * 64]
    rng = np.random.default_rng(23)
    lens += [int(x) for x in rng.integers(0, maxp * 64 + 1, B - len(lens))]
    L, cache, table, kv, g = _setup(lens, "fp4", seed=25, maxp=maxp)
    q = torch.randn(B, HKV * G, D, generator=g).to(torch.bfloat16)
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    _say(f"window {window}: chunks {tuple(ch)}, promised the whole table {tuple(ch_h)}")
    outs = [fk.decode_with_options(L, cache, q.cuda(), lens_d, table.cuda(), window=window, num_splits=splits,
                                   min_seq_len=m).cpu().numpy() for m in (0, maxp * 64)]
    worst = 0.0
    for b, n in enumerate(lens):
        if n == 0:
            assert not outs[0][b].any() and not outs[1][b].any()
            continue
        lo = max(0, n - window)
        kq = oracle.quantize(wl.bf16_bits(kv[b][0][lo:n]), want_xhat=False)
        vq = oracle.quantize(wl.bf16_bits(kv[b][1][lo:n]), want_xhat=False)
        r = oracle.decode_attention(wl.bf16_bits(q[b:b + 1]), [kq[0]], [kq[1]], [vq[0]], [vq[1]], [n - lo],
                                    D ** -0.5)
        for o in outs:
            worst = max(worst, float(hx.row_rel_error(o[b][None], r).max()))
    _say(f"  worst per-row relative error (both cuts) {worst:.3e}")
    assert worst <= TOL
