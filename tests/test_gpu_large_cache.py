"""Caches past 2^32 bytes: every byte offset the kernels form must be 64-bit.

- An FP4 pool of 60,000 pages x 8 KV heads (4.4 GB): three sequences whose
  pages lie at the top of the pool, straddle the 2^32-byte mark, or
  alternate between its two ends.  Appended through fp4kv_quantize_append
  and, one more token each, through the decode step that stores its own
  token; the stored bytes of every used page must equal the oracle's codes,
  and decode attention through every split kernel must be within 1e-3 per
  row of the oracle's.
- The same for an FP8 (per-tensor scale) pool of 35,000 pages (4.6 GB).
- A bf16 tensor of the bit-width sweep's head-major layout holding 2.25 GB
  per tensor (one sequence, 16 KV heads, 550,000 tokens): decode attention
  of the last KV head, whose rows start past 2^31 bytes, against the oracle.
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
H, D, G = 8, 128, 8


def _say(msg):
    print(msg, flush=True)


def _page_lists(num_pages):
    """Per sequence: (length, its pages in order)."""
    top = list(range(num_pages - 63, num_pages))                     # the last 63 pages
    mark = 2 ** 32 // (H * 9216) - 1                                 # FP4: a page around the 2^32-byte mark
    alternate = [j // 2 if j % 2 == 0 else num_pages - 100 - j for j in range(47)]
    return [(4000, top), (2 * 64 + 17, list(range(mark - 1, mark + 2))), (3000, alternate)]


def _rows(n, seed):
    g = torch.Generator().manual_seed(seed)
    f = torch.exp(torch.empty(H, D).uniform_(-1.5, 1.5, generator=g))
    return (torch.randn(n, H, D, generator=g) * f).to(torch.bfloat16)


def _slots(pages, t0, t1):
    return torch.tensor([pages[t // 64] * 64 + t % 64 for t in range(t0, t1)], dtype=torch.int64)


def _build(layout, seqs, seed):
    cache = torch.empty(layout.cache_bytes, dtype=torch.uint8, device="cuda")
    assert layout.cache_bytes > 2 ** 32
    rows = []
    for i, (n, pages) in enumerate(seqs):
        k, v = _rows(n + 1, seed + 2 * i), _rows(n + 1, seed + 2 * i + 1)      # + the step's token
        fk.quantize_append(layout, k[:n].cuda(), v[:n].cuda(), _slots(pages, 0, n).cuda(), cache)
        rows.append((k, v))
    maxp = max(len(p) for _, p in seqs)
    table = torch.zeros(len(seqs), maxp, dtype=torch.int32)
    for i, (_, pages) in enumerate(seqs):
        table[i, :len(pages)] = torch.tensor(pages, dtype=torch.int32)
    torch.cuda.synchronize()
    return cache, rows, table.cuda()


def _check(layout, cache, seqs, rows, table, lens, fmt):
    """Stored bytes of every used page and decode through every kernel."""
    q = torch.randn(len(seqs), H * G, D, generator=torch.Generator().manual_seed(7)).to(torch.bfloat16)
    kc, ks, vc, vs = [], [], [], []
    for (n, pages), (k, v), L in zip(seqs, rows, lens):
        kb, vb = wl.bf16_bits(k[:L]), wl.bf16_bits(v[:L])
        if fmt == "fp4":
            gk, gks, gv, gvs = hx.read_pages(cache, layout, pages, L)
            (okn, oks, _), (ovn, ovs, _) = oracle.quantize(kb, want_xhat=False), oracle.quantize(vb, want_xhat=False)
            assert np.array_equal(gk, oracle.pack_nibbles(okn)) and np.array_equal(gks, oks)
            assert np.array_equal(gv, oracle.pack_nibbles(ovn)) and np.array_equal(gvs, ovs)
            kc.append(okn); ks.append(oks); vc.append(ovn); vs.append(ovs)
        else:
            gk, gv = hx.read_pages_fp8(cache, layout, pages, L)
            ok_, ov_ = oracle.quantize_fp8(kb, layout.params.k_scale), oracle.quantize_fp8(vb, layout.params.v_scale)
            assert np.array_equal(gk, ok_) and np.array_equal(gv, ov_)
            kc.append(ok_); vc.append(ov_)
    if fmt == "fp4":
        ref = oracle.decode_attention(wl.bf16_bits(q), kc, ks, vc, vs, lens, D ** -0.5)
        kernels = ("auto", "mfma_direct", "valu")
    else:
        ref = oracle.decode_attention_fp8(wl.bf16_bits(q), kc, vc, layout.params.k_scale, layout.params.v_scale,
                                          lens, D ** -0.5)
        kernels = ("auto",)
    seq_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for kern in kernels:
        for splits in (0, 1):
            out = fk.decode_with_options(layout, cache, q.cuda(), seq_lens, table, num_splits=splits, kernel=kern)
            torch.cuda.synchronize()
            err = float(hx.row_rel_error(out.cpu().numpy(), ref).max())
            _say(f"  {fmt} kernel {kern}, splits {splits}: worst per-row relative error {err:.3e}")
            assert err <= TOL


@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_pool_past_4gib(fmt):
    if fmt == "fp4":
        layout = fk.cache_layout(H, D, 60000)
    else:
        layout = fk.cache_layout(H, D, 35000, format=fk.FORMAT_FP8_E4M3, k_scale=0.03, v_scale=0.02)
    seqs = _page_lists(layout.num_pages)
    if fmt == "fp8":            # the FP8 page is larger: move the middle sequence to its own 2^32-byte mark
        mark = 2 ** 32 // layout.block_bytes // H - 1
        seqs[1] = (seqs[1][0], list(range(mark - 1, mark + 2)))
    _say(f"{fmt} pool of {layout.num_pages} pages, {layout.cache_bytes / 2 ** 30:.2f} GiB")
    cache, rows, table = _build(layout, seqs, seed=11)
    lens = [n for n, _ in seqs]
    _check(layout, cache, seqs, rows, table, lens, fmt)
    # one decode step that stores each sequence's next token itself
    k_new = torch.stack([k[n] for (n, _), (k, _) in zip(seqs, rows)]).cuda()
    v_new = torch.stack([v[n] for (n, _), (_, v) in zip(seqs, rows)]).cuda()
    q = torch.randn(len(seqs), H * G, D, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    lens1 = [n + 1 for n in lens]
    fk.decode_append_attention(layout, cache, k_new, v_new, q.cuda(),
                               torch.tensor(lens1, dtype=torch.int32, device="cuda"), table)
    torch.cuda.synchronize()
    _say(f"  {fmt}: after the decode step that appends one token per sequence")
    _check(layout, cache, seqs, rows, table, lens1, fmt)


def test_sweep_tensor_past_2gib():
    B, Hs, T, Gs = 1, 16, 550000, 4
    g = torch.Generator(device="cuda").manual_seed(5)
    x_k = torch.randn(B, T, Hs, D, generator=g, device="cuda").to(torch.bfloat16)
    x_v = torch.randn(B, T, Hs, D, generator=g, device="cuda").to(torch.bfloat16)
    q = torch.randn(B, Hs * Gs, D, generator=g, device="cuda").to(torch.bfloat16)
    kq, vq = fk.int_quantize(x_k, 16), fk.int_quantize(x_v, 16)
    assert kq[0].numel() > 2 ** 31
    _say(f"sweep bf16 tensor of {kq[0].numel() / 2 ** 30:.2f} GiB: decode, last KV head")
    out = fk.int_decode_attention(q, 16, kq, vq, T)
    torch.cuda.synchronize()
    h = Hs - 1
    kv = oracle.bf16_values(wl.bf16_bits(x_k[0, :, h:h + 1].cpu()))          # [T][1][D]
    vv = oracle.bf16_values(wl.bf16_bits(x_v[0, :, h:h + 1].cpu()))
    qh = q[:, h * Gs:(h + 1) * Gs].cpu()
    ref = oracle.decode_attention_values(wl.bf16_bits(qh), [kv], [vv], [T], D ** -0.5)
    err = float(hx.row_rel_error(out[:, h * Gs:(h + 1) * Gs].cpu().numpy(), ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL
