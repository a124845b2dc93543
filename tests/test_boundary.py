"""The C ABI on the CPU: the library loads, exports what include/*.h
declares, and every host-side check fires before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

import fp4_quantised_kv_amd as fk
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    return sorted(set(re.findall(r"FP4KV_API\s+[\w\s\*]*?\b(fp4kv_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"fp4kv_cache_layout", "fp4kv_quantize_append", "fp4kv_decode_attention",
            "fp4kv_int_quantize", "fp4kv_int_decode_attention"} <= set(names)
    lib = fk.library()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert fk.library().fp4kv_version() == fk.VERSION == 200
    for code in (0, -1, -2, -3, -4, -5):
        assert fk.status_string(code) not in ("", "unknown status")
    assert fk.status_string(-99) == "unknown status"


@pytest.mark.parametrize("H,D,pages", [(1, 64, 4), (8, 128, 512), (8, 128, 1), (3, 64, 1000)])
def test_layout_sizes(H, D, pages):
    L = fk.cache_layout(H, D, pages)
    assert L.block_bytes == 64 * D * 9 // 8
    assert L.cache_bytes == pages * H * L.block_bytes
    # 4.5 bits per number, exactly: the cost the oracle's cost model gives
    assert L.cache_bytes == oracle.fp4_cache_bytes(pages * 64, 1, H, D)
    assert L.bytes_per_token * 64 * pages == L.cache_bytes
    offs = [L.k_codes_offset, L.k_scales_offset, L.v_codes_offset, L.v_scales_offset]
    sizes = [64 * D // 2, 64 * D // 16, 64 * D // 2, 64 * D // 16]
    assert offs == [0, sizes[0], sizes[0] + sizes[1], sizes[0] + sizes[1] + sizes[2]]
    assert all(o % 16 == 0 for o in offs) and L.block_bytes % 256 == 0
    assert L.page_stride == H * L.block_bytes and L.head_stride == L.block_bytes


@pytest.mark.parametrize("H,D,P,pages,fmt,ks,vs,code", [
    (0, 128, 64, 1, 0, 0, 0, fk.ERR_INVALID_ARGUMENT), (8, 128, 64, 0, 0, 0, 0, fk.ERR_INVALID_ARGUMENT),
    (8, 128, 64, 1, 3, 0, 0, fk.ERR_INVALID_ARGUMENT), (8, 96, 64, 1, 0, 0, 0, fk.ERR_UNSUPPORTED),
    (8, 100, 64, 1, 0, 0, 0, fk.ERR_UNSUPPORTED), (8, 256, 64, 1, 0, 0, 0, fk.ERR_UNSUPPORTED),
    (8, 128, 32, 1, 0, 0, 0, fk.ERR_UNSUPPORTED), (8, 128, 64, 1 << 60, 0, 0, 0, fk.ERR_INVALID_ARGUMENT),
    (8, 128, 64, 1, 0, 1.0, 0, fk.ERR_INVALID_ARGUMENT),            # FP4 takes no scales
    (8, 128, 64, 1, 1, 0.0, 1.0, fk.ERR_INVALID_ARGUMENT),          # FP8 needs both scales
    (8, 128, 64, 1, 1, 1.0, -1.0, fk.ERR_INVALID_ARGUMENT),
    (8, 128, 64, 1, 1, float("inf"), 1.0, fk.ERR_INVALID_ARGUMENT),
    (8, 128, 64, 1, 1, 1.0, float("nan"), fk.ERR_INVALID_ARGUMENT),
    (8, 128, 64, 1, 1, 2.0 ** -70, 1.0, fk.ERR_UNSUPPORTED),        # outside 2^-64 .. 2^64
    (8, 128, 64, 1, 1, 1.0, 2.0 ** 70, fk.ERR_UNSUPPORTED),
    (8, 96, 64, 1, 1, 1.0, 1.0, fk.ERR_UNSUPPORTED),                # FP8: D 64 or 128 too
    (8, 96, 64, 1, 2, 0.0, 0.0, fk.ERR_UNSUPPORTED)])
def test_layout_rejects(H, D, P, pages, fmt, ks, vs, code):
    p = fk.CacheParams(H, D, P, fmt, pages, ks, vs)
    out = fk.CacheLayout()
    assert fk.library().fp4kv_cache_layout(ctypes.byref(p), ctypes.byref(out)) == code
    assert fk.library().fp4kv_cache_layout(None, ctypes.byref(out)) == fk.ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("H,pages", [(1, 1), (8, 512), (3, 1000)])
def test_fp8_layout_sizes(H, pages):
    L64 = fk.cache_layout(H, 64, pages, format=fk.FORMAT_FP8_E4M3, k_scale=0.5, v_scale=3.0)
    assert L64.block_bytes == 64 * 64 * 2 and L64.v_codes_offset == 64 * 64
    L = fk.cache_layout(H, 128, pages, format=fk.FORMAT_FP8_E4M3, k_scale=0.5, v_scale=3.0)
    assert L.block_bytes == 64 * 128 * 2 and L.fp8
    # 8 bits per number, exactly: the oracle's cost model for FP8 with one scale per tensor
    assert L.cache_bytes == pages * H * L.block_bytes == oracle.fp8_cache_bytes(pages * 64, 1, H, 128)
    assert [L.k_codes_offset, L.k_scales_offset, L.v_codes_offset, L.v_scales_offset] == [0, 8192, 8192, 16384]
    assert L.bytes_per_token * 64 == L.page_stride == H * L.block_bytes
    assert (L.params.k_scale, L.params.v_scale) == (0.5, 3.0)


@pytest.mark.parametrize("H,D,pages", [(1, 64, 1), (8, 128, 512), (3, 128, 1000)])
def test_fp8_token_layout_sizes(H, D, pages):
    """FP8 with an fp16 scale per (token, KV head): K codes, K scales, V
    codes, V scales per block; 8 + 16/D bits per number, the page's cost
    formula b + s/g with s = 16 and g = D."""
    L = fk.cache_layout(H, D, pages, format=fk.FORMAT_FP8_E4M3_TOKEN)
    assert L.block_bytes == 128 * D + 256 and L.fp8 and L.token_scales
    assert [L.k_codes_offset, L.k_scales_offset, L.v_codes_offset, L.v_scales_offset] == \
        [0, 64 * D, 64 * D + 128, 128 * D + 128]
    assert 8 * L.cache_bytes / (pages * 64 * 2 * H * D) == pytest.approx(oracle.bits_per_number(8, 16, D))
    assert L.bytes_per_token * 64 == L.page_stride == H * L.block_bytes
    for ks, vs in ((0.5, 0.0), (0.0, 1.0)):                       # it takes no tensor scales
        p = fk.CacheParams(H, D, 64, fk.FORMAT_FP8_E4M3_TOKEN, pages, ks, vs)
        assert fk.library().fp4kv_cache_layout(ctypes.byref(p), ctypes.byref(fk.CacheLayout())) == \
            fk.ERR_INVALID_ARGUMENT
    p = fk.CacheParams(H, D, 64, 3, pages, 0.0, 0.0)                # unknown format
    assert fk.library().fp4kv_cache_layout(ctypes.byref(p), ctypes.byref(fk.CacheLayout())) == \
        fk.ERR_INVALID_ARGUMENT


def test_plan():
    L = fk.cache_layout(8, 128, 32 * 512)
    assert fk.decode_plan(L, 32, 64, 512, 64)[:2] == (64, 16)       # four chunks per workgroup
    assert fk.decode_plan(L, 32, 64, 512, 64)[2] == 32 * 64 * 16 * 128 * 4 + 32 * 64 * 16 * 8
    assert fk.decode_plan(L, 1, 32, 8192, 7).partials == 2
    assert fk.decode_plan(L, 1, 32, 8192, 256)[0] == 256
    assert fk.decode_plan(L, 1, 32, 3, 256)[0] == 3                 # never more splits than pages
    assert fk.decode_plan(L, 1, 32, 10, 4)[0] == 4                  # 3 pages per split: 4 splits
    assert fk.decode_plan(L, 1, 32, 9, 4)[0] == 3                   # 3 pages per split: 3 splits
    s, p, ws = fk.decode_plan(L, 64, 32, 258, 0)
    assert 1 <= s <= 258 and p == -(-s // 4) and ws > 0
    # the automatic choice keeps chunks of at least two pages while 1024 chunks remain
    assert fk.decode_plan(L, 8, 32, 64, 0)[:2] == (32, 8)           # 8 x 8 x 32 = 2048 chunks
    assert fk.decode_plan(L, 1, 32, 64, 0)[0] == 64                 # 8 x 32 < 1024: one page each
    assert fk.decode_plan(L, 1, 32, 3, 0)[0] == 3
    assert fk.decode_plan(L, 1, 32, 1, 0)[0] == 1
    assert fk.decode_plan(L, 64, 32, 258, 0)[0] == 29               # the ragged paged batch: 9 pages a chunk
    for args, code in [((32, 65, 512, 64), fk.ERR_INVALID_ARGUMENT),      # Hq % Hkv
                       ((32, 8 * 17, 512, 64), fk.ERR_UNSUPPORTED),       # group 17
                       ((-1, 64, 512, 64), fk.ERR_INVALID_ARGUMENT),
                       ((1, 64, 0, 64), fk.ERR_INVALID_ARGUMENT),
                       ((1, 64, 8, -1), fk.ERR_INVALID_ARGUMENT)]:
        with pytest.raises(fk.Fp4KVError) as e:
            fk.decode_plan(L, *args)
        assert e.value.status == code


def test_chunks():
    L = fk.cache_layout(8, 128, 32 * 512)
    # 8 x 32 x 16 = 4096 workgroups: the last 8 partials take chunks of
    # 3 pages (3/8 of 8), the first 32 chunks share out the other 416 pages
    assert tuple(fk.decode_chunks(L, 32, 64, 512, 64)) == (32, 13, 3)
    # the paged batch: 29 chunks of 9 pages in 8 partials, 4096 workgroups
    assert tuple(fk.decode_chunks(L, 64, 32, 258, 0)) == (16, 14, 3)
    # fewer than 1536 workgroups: even chunks
    assert tuple(fk.decode_chunks(L, 1, 32, 8192, 256)) == (256, 32, 32)
    assert tuple(fk.decode_chunks(L, 8, 32, 64, 0)) == (32, 2, 2)
    assert tuple(fk.decode_chunks(L, 8, 32, 64, 0, q_tokens=2, window=0)) == (32, 2, 2)
    for B, Hq, maxp, S, qt, win in [(32, 64, 512, 64, 1, 0), (64, 32, 258, 0, 1, 0), (48, 32, 48, 16, 1, 0),
                                    (64, 32, 48, 16, 1, 0), (96, 32, 32, 7, 2, 700), (96, 32, 32, 0, 2, 700),
                                    (200, 8, 100, 3, 1, 0), (6, 8, 5000, 0, 1, 0), (512, 64, 40, 40, 1, 0),
                                    (33, 16, 77, 29, 4, 300), (1024, 8, 2, 0, 1, 0)]:
        span = maxp if win == 0 else min(maxp, -(-(win + qt - 1) // 64) + 1)
        plan = (fk.decode_plan(L, B, Hq, maxp, S) if win == 0 and qt == 1
                else fk.decode_window_plan(L, B, qt, Hq, maxp, win, S))
        ch = fk.decode_chunks(L, B, Hq, maxp, S, q_tokens=qt, window=win)
        pps = -(-span // plan.splits)
        chunks = 4 * plan.partials
        assert ch.first_page(chunks) >= span                          # the chunks tile the span
        if ch.lead_chunks == chunks:
            assert ch.lead_pages == ch.tail_pages == pps
        else:
            assert 8 * B * plan.partials >= 1536
            assert ch.lead_chunks == 4 * (plan.partials - plan.partials // 2)
            assert ch.tail_pages == max(1, 3 * pps // 8) < pps <= ch.lead_pages
            # the lead chunks hold no more than they must: a page fewer each leaves pages uncovered
            assert ch.lead_chunks * (ch.lead_pages - 1) + (chunks - ch.lead_chunks) * ch.tail_pages < span
    for kw, code in [(dict(q_tokens=0), fk.ERR_INVALID_ARGUMENT), (dict(window=-1), fk.ERR_INVALID_ARGUMENT)]:
        with pytest.raises(fk.Fp4KVError) as e:
            fk.decode_chunks(L, 4, 32, 16, 0, **kw)
        assert e.value.status == code
    for args, code in [((32, 65, 512, 64), fk.ERR_INVALID_ARGUMENT), ((1, 64, 0, 64), fk.ERR_INVALID_ARGUMENT),
                       ((32, 8 * 17, 512, 64), fk.ERR_UNSUPPORTED)]:
        with pytest.raises(fk.Fp4KVError) as e:
            fk.decode_chunks(L, *args)
        assert e.value.status == code
    lc = ctypes.c_int32()
    assert fk.library().fp4kv_decode_chunks(ctypes.byref(L), 4, 1, 32, 16, 0, 0, 0, ctypes.byref(lc), None,
                                            ctypes.byref(lc)) == fk.ERR_INVALID_ARGUMENT


def test_chunks_with_a_shortest_length():
    """min_seq_len: when every sequence covers at least 7/8 of the span,
    every partial after the lead ones takes chunks of 1/8 of the even size
    (at least a page); the lead partials are the fewest whose workgroups
    fill 768 resident slots for the FP4 cache, a quarter of the partials (or
    that many) for the FP8 caches.  A smaller bound, or none, keeps the
    default cut."""
    L = fk.cache_layout(8, 128, 32 * 512)
    # the 32 x 32K batch at 64 chunks: 3 lead partials (3 x 256 = 768 workgroups)
    # of 39-page chunks, then 52 one-page chunks
    assert tuple(fk.decode_chunks(L, 32, 64, 512, 64, min_seq_len=32768)) == (12, 39, 1)
    assert tuple(fk.decode_chunks(L, 32, 64, 512, 64, min_seq_len=7 * 512 * 64 // 8)) == (12, 39, 1)
    assert tuple(fk.decode_chunks(L, 32, 64, 512, 64, min_seq_len=7 * 512 * 64 // 8 - 64)) == (32, 13, 3)
    # 64 sequences: one partial is 512 workgroups, so two lead partials
    assert tuple(fk.decode_chunks(L, 64, 64, 512, 64, min_seq_len=32768)) == (8, 57, 1)
    # the FP8 caches keep a quarter of the partials as lead ones (16 chunks of 29 pages, 48 of
    # one), or more where a quarter would not fill the GPU (16 sequences: 6 partials of 128)
    for kw in (dict(format=fk.FORMAT_FP8_E4M3, k_scale=1.0, v_scale=1.0), dict(format=fk.FORMAT_FP8_E4M3_TOKEN)):
        L8 = fk.cache_layout(8, 128, 32 * 512, **kw)
        assert tuple(fk.decode_chunks(L8, 32, 64, 512, 64, min_seq_len=32768)) == (16, 29, 1)
        assert tuple(fk.decode_chunks(L8, 16, 64, 512, 64, min_seq_len=32768)) == (24, 20, 1)
        assert tuple(fk.decode_chunks(L8, 32, 64, 512, 64)) == (32, 13, 3)
    # the paged batch's shortest sequence (1,024 tokens) keeps the default cut
    assert tuple(fk.decode_chunks(L, 64, 32, 258, 0, min_seq_len=1024)) == (16, 14, 3)
    # fewer than 1536 workgroups: even chunks whatever the bound
    assert tuple(fk.decode_chunks(L, 1, 32, 8192, 256, min_seq_len=8192 * 64)) == (256, 32, 32)
    for B, Hq, maxp, S, qt, win in [(32, 64, 512, 64, 1, 0), (64, 32, 258, 0, 1, 0), (48, 32, 48, 16, 1, 0),
                                    (64, 32, 48, 16, 1, 0), (96, 32, 32, 7, 2, 700), (96, 32, 32, 0, 2, 700),
                                    (200, 8, 100, 3, 1, 0), (512, 64, 40, 40, 1, 0), (33, 16, 77, 29, 4, 300),
                                    (1024, 8, 2, 0, 1, 0), (64, 32, 400, 32, 1, 0), (128, 64, 300, 64, 1, 0)]:
        span = maxp if win == 0 else min(maxp, -(-(win + qt - 1) // 64) + 1)
        plan = (fk.decode_plan(L, B, Hq, maxp, S) if win == 0 and qt == 1
                else fk.decode_window_plan(L, B, qt, Hq, maxp, win, S))
        pps = -(-span // plan.splits)
        chunks = 4 * plan.partials
        for min_len in (span * 64, maxp * 64, -(-7 * span // 8) * 64):
            ch = fk.decode_chunks(L, B, Hq, maxp, S, q_tokens=qt, window=win, min_seq_len=min_len)
            assert ch.first_page(chunks) >= span                      # the chunks tile the span
            if ch.lead_chunks == chunks:
                assert ch.lead_pages == ch.tail_pages == pps
            else:
                assert 8 * B * plan.partials >= 1536
                assert ch.lead_chunks == 4 * -(-768 // (8 * B))
                assert ch.tail_pages == max(1, pps // 8) < pps <= ch.lead_pages
                assert ch.lead_chunks * (ch.lead_pages - 1) + (chunks - ch.lead_chunks) * ch.tail_pages < span
        # a bound under 7/8 of the span: the default cut
        assert fk.decode_chunks(L, B, Hq, maxp, S, q_tokens=qt, window=win,
                                min_seq_len=(7 * span // 8 - 1) * 64) == fk.decode_chunks(L, B, Hq, maxp, S,
                                                                                         q_tokens=qt, window=win)
    with pytest.raises(fk.Fp4KVError) as e:
        fk.decode_chunks(L, 4, 32, 16, 0, min_seq_len=-1)
    assert e.value.status == fk.ERR_INVALID_ARGUMENT


def _lib():
    return fk.library()


def test_quantize_append_host_checks():
    L = fk.cache_layout(8, 128, 4)
    lib = _lib()
    ok = 0x10000                                        # aligned fake device addresses: never
    assert lib.fp4kv_quantize_append(ctypes.byref(L), ok, ok, 0, ok, ok, None) == fk.OK
    assert lib.fp4kv_quantize_append(ctypes.byref(L), ok, ok, -1, ok, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_quantize_append(ctypes.byref(L), None, ok, 5, ok, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_quantize_append(ctypes.byref(L), ok, ok, 5, None, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_quantize_append(ctypes.byref(L), ok + 8, ok, 5, ok, ok, None) == fk.ERR_MISALIGNED
    assert lib.fp4kv_quantize_append(ctypes.byref(L), ok, ok, 5, ok + 4, ok, None) == fk.ERR_MISALIGNED
    assert lib.fp4kv_quantize_append(ctypes.byref(L), ok, ok, 5, ok, ok + 16, None) == fk.ERR_MISALIGNED
    assert lib.fp4kv_quantize_append(None, ok, ok, 5, ok, ok, None) == fk.ERR_INVALID_ARGUMENT
    bad = fk.CacheLayout.from_buffer_copy(L)
    bad.cache_bytes += 1                                # not what fp4kv_cache_layout produced
    assert lib.fp4kv_quantize_append(ctypes.byref(bad), ok, ok, 5, ok, ok, None) == fk.ERR_INVALID_ARGUMENT


def test_decode_host_checks():
    L = fk.cache_layout(8, 128, 64)
    lib = _lib()
    ok = 0x10000
    s, p, ws = fk.decode_plan(L, 2, 32, 8, 0)

    def call(**kw):
        a = dict(cache=ok, q=ok, batch=2, hq=32, lens=ok, pt=ok, maxp=8, scale=0.1, splits=0,
                 ws=ok, wsb=ws, out=ok)
        a.update(kw)
        return lib.fp4kv_decode_attention(ctypes.byref(L), a["cache"], a["q"], a["batch"], a["hq"],
                                          a["lens"], a["pt"], a["maxp"], a["scale"], a["splits"],
                                          a["ws"], a["wsb"], a["out"], None)

    assert call(batch=0) == fk.OK
    assert call(cache=None) == fk.ERR_INVALID_ARGUMENT
    assert call(out=None) == fk.ERR_INVALID_ARGUMENT
    assert call(hq=33) == fk.ERR_INVALID_ARGUMENT
    assert call(hq=8 * 32) == fk.ERR_UNSUPPORTED
    assert call(scale=float("nan")) == fk.ERR_INVALID_ARGUMENT
    assert call(scale=0.0) == fk.ERR_INVALID_ARGUMENT
    assert call(scale=-0.1) == fk.ERR_INVALID_ARGUMENT
    assert call(q=ok + 2) == fk.ERR_MISALIGNED
    assert call(ws=ok + 64) == fk.ERR_MISALIGNED
    assert call(cache=ok + 128) == fk.ERR_MISALIGNED
    assert call(out=ok + 4) == fk.ERR_MISALIGNED
    assert call(wsb=ws - 1) == fk.ERR_WORKSPACE_TOO_SMALL
    assert call(batch=70000) == fk.ERR_UNSUPPORTED
    assert lib.fp4kv_decode_combine(2, 32, 128, 0, ok, ws, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_decode_combine(2, 32, 96, 4, ok, ws, ok, None) == fk.ERR_UNSUPPORTED
    assert lib.fp4kv_decode_combine(2, 32, 128, p, ok, ws - 1, ok, None) == fk.ERR_WORKSPACE_TOO_SMALL
    assert lib.fp4kv_decode_combine(0, 32, 128, p, None, 0, None, None) == fk.OK
    assert lib.fp4kv_decode_split(ctypes.byref(L), ok, ok, 2, 32, ok, ok, 8, 0.1, 0, ok, ws - 1,
                                  None) == fk.ERR_WORKSPACE_TOO_SMALL


def test_binding_refuses_cpu_tensors():
    import torch
    L = fk.cache_layout(1, 64, 1)
    k = torch.zeros(1, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fk.quantize_append(L, k, k, torch.zeros(1, dtype=torch.int64),
                           torch.zeros(L.cache_bytes, dtype=torch.uint8))


def test_read_probe_host_checks():
    lib = _lib()
    ok = 0x10000
    assert lib.fp4kv_read_probe(None, 9216, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_read_probe(ok, 0, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_read_probe(ok, 9215, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_read_probe(ok, 9216, None, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_read_probe(ok + 16, 9216, ok, None) == fk.ERR_MISALIGNED
    assert lib.fp4kv_read_probe(ok, 9216, ok + 2, None) == fk.ERR_MISALIGNED
    cfg = lib.fp4kv_read_probe_config
    assert cfg(None, 16384, 16, 256, 0, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert cfg(ok, 16384, 3, 256, 0, ok, None) == fk.ERR_INVALID_ARGUMENT      # loads per lane 1, 2, 4, 8, 16
    assert cfg(ok, 16384 + 1024, 16, 256, 0, ok, None) == fk.ERR_INVALID_ARGUMENT   # whole stretches
    assert cfg(ok, 16384, 16, 0, 0, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert cfg(ok, 16384, 16, 256, 2, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert cfg(ok + 512, 16384, 16, 256, 0, ok, None) == fk.ERR_MISALIGNED
    assert cfg(ok, 16384, 16, 256, 1, ok + 1, None) == fk.ERR_MISALIGNED
    sp = lib.fp4kv_stream_probe
    assert sp(None, ok, 4, 8192, 1024, 0, 256, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert sp(ok, ok, 0, 8192, 1024, 0, 256, ok, None) == fk.ERR_INVALID_ARGUMENT      # no units
    assert sp(ok, ok, 4, 4096, 1024, 0, 256, ok, None) == fk.ERR_INVALID_ARGUMENT      # reads in 8 KB steps
    assert sp(ok, ok, 4, 8192, 1000, 0, 256, ok, None) == fk.ERR_INVALID_ARGUMENT      # writes in 1 KB steps
    assert sp(ok, None, 4, 8192, 1024, 0, 256, ok, None) == fk.ERR_INVALID_ARGUMENT    # writes need dst
    assert sp(ok, ok, 4, 8192, 1024, 2, 256, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert sp(ok, ok, 4, 8192, 1024, 0, 0, ok, None) == fk.ERR_INVALID_ARGUMENT
    assert sp(ok, ok, 4, 8192, 1024, 0, 256, None, None) == fk.ERR_INVALID_ARGUMENT
    assert sp(ok + 16, ok, 4, 8192, 1024, 0, 256, ok, None) == fk.ERR_MISALIGNED
    assert sp(ok, ok + 16, 4, 8192, 1024, 1, 256, ok, None) == fk.ERR_MISALIGNED
    assert sp(ok, ok, 4, 8192, 1024, 1, 256, ok + 2, None) == fk.ERR_MISALIGNED


# ------------------------------------------------ integer formats (fp4kv_int.h)

@pytest.mark.parametrize("B,T,H,D,bits,gran", [(2, 100, 3, 128, 8, "token"), (1, 7, 1, 64, 4, "channel"),
                                               (4, 33, 8, 128, 2, "token"), (2, 5, 2, 64, 16, "channel"),
                                               (2, 100, 3, 128, fk.INT_FP8_E4M3, "token"),
                                               (3, 9, 2, 64, fk.INT_FP8_E4M3, "channel")])
def test_int_sizes(B, T, H, D, bits, gran):
    nc, ns = fk.int_sizes(B, T, H, D, bits, gran)
    if bits == fk.INT_FP8_E4M3:
        bits = 8                                        # one E4M3 byte per number, fp16 scales as INT8
    assert nc == B * T * H * D * bits // 8
    if bits == 16:
        assert ns == 0
    elif gran == "token":
        assert ns == B * T * H * 2
    else:
        assert ns == B * H * D * 2
    # bits per number b + 16/g with g = D (per token) or T (per channel)
    if bits != 16:
        per = (8 * (nc + ns)) / (B * T * H * D)
        g = D if gran == "token" else T
        assert per == pytest.approx(oracle.bits_per_number(bits, 16, g))


@pytest.mark.parametrize("args,code", [
    ((1, 4, 1, 128, 3, 0), fk.ERR_INVALID_ARGUMENT), ((1, 4, 1, 128, 8, 2), fk.ERR_INVALID_ARGUMENT),
    ((1, 4, 0, 128, 8, 0), fk.ERR_INVALID_ARGUMENT), ((-1, 4, 1, 128, 8, 0), fk.ERR_INVALID_ARGUMENT),
    ((1, -4, 1, 128, 8, 0), fk.ERR_INVALID_ARGUMENT), ((1, 4, 1, 96, 8, 0), fk.ERR_UNSUPPORTED),
    ((1, 4, 1, 128, 0x109, 0), fk.ERR_INVALID_ARGUMENT), ((1, 4, 1, 128, 0x108, 3), fk.ERR_INVALID_ARGUMENT)])
def test_int_sizes_rejects(args, code):
    with pytest.raises(fk.Fp4KVError) as e:
        fk.int_sizes(*args)
    assert e.value.status == code


def test_int_plan_and_workspace():
    # T = 1000 tokens: 4 chunks of 256; ask for 3 splits -> 2 chunks each -> 2 splits
    s, ws = fk.int_decode_plan(2, 1000, 4, 128, 16, 3)
    assert s == 2
    rows = 2 * 16 * s
    assert ws == -(-rows * 128 * 4 // 256) * 256 + -(-rows * 8 // 256) * 256
    assert fk.int_decode_plan(2, 1000, 4, 128, 16, 100)[0] == 4       # clamped to the chunks
    assert fk.int_decode_plan(2, 0, 4, 128, 16, 0)[0] == 1            # empty context: one empty split
    auto = fk.int_decode_plan(8, 4096, 8, 128, 32, 0)[0]
    assert 1 <= auto <= 16 and 8 * 8 * auto >= 512
    for bad, code in (((2, 1000, 4, 128, 6, 0), fk.ERR_INVALID_ARGUMENT),      # 6 % 4
                      ((2, 1000, 1, 128, 17, 0), fk.ERR_UNSUPPORTED),          # group of 17
                      ((2, 1000, 4, 128, 16, -1), fk.ERR_INVALID_ARGUMENT)):
        with pytest.raises(fk.Fp4KVError) as e:
            fk.int_decode_plan(*bad)
        assert e.value.status == code


def test_int_calls_reject_before_any_hip_call():
    L = fk.library()
    d = fk.IntDims(1, 16, 1, 128)
    # null data pointers, misalignment and a small workspace are refused on the host
    assert L.fp4kv_int_quantize(ctypes.byref(d), 8, 0, None, None, None, None) == fk.ERR_INVALID_ARGUMENT
    assert L.fp4kv_int_quantize(ctypes.byref(d), 8, 0, 16, 32, 49, None) == fk.ERR_MISALIGNED
    assert L.fp4kv_int_quantize(ctypes.byref(d), 5, 0, 16, 32, 48, None) == fk.ERR_INVALID_ARGUMENT
    z = fk.IntDims(0, 16, 1, 128)
    assert L.fp4kv_int_quantize(ctypes.byref(z), 8, 0, None, None, None, None) == fk.OK   # nothing to do
    args = [ctypes.byref(d), 8, 0, 0, 256, 512, 256, 512, 256, 1, ctypes.c_float(0.1), 0, 256]
    assert L.fp4kv_int_decode_attention(*args, 10, 256, None) == fk.ERR_WORKSPACE_TOO_SMALL
    args[10] = ctypes.c_float(0.0)
    assert L.fp4kv_int_decode_attention(*args, 1 << 20, 256, None) == fk.ERR_INVALID_ARGUMENT
    args[10] = ctypes.c_float(0.1)
    args[4] = 264                                       # k codes not 16-B aligned
    assert L.fp4kv_int_decode_attention(*args, 1 << 20, 256, None) == fk.ERR_MISALIGNED


def test_append_decode_rejects_missing_or_misaligned_rows():
    """fp4kv_decode_append_attention checks the new-token rows on the host
    (the other arguments are valid, aligned stand-ins; nothing is launched)."""
    L = fk.cache_layout(1, 128, 4)
    lib = fk.library()
    args = lambda kn: (ctypes.byref(L), 256, kn, 256, 256, 1, 4, 256, 256, 4, ctypes.c_float(0.1), 0, 256,
                       1 << 20, 256, None)
    assert lib.fp4kv_decode_append_attention(*args(None)) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_decode_append_attention(*args(264)) == fk.ERR_MISALIGNED
    assert lib.fp4kv_decode_append_split(*args(None)[:-2], None) == fk.ERR_INVALID_ARGUMENT


def test_window_rejects_negative_window():
    L = fk.cache_layout(2, 128, 16)
    with pytest.raises(fk.Fp4KVError) as e:
        fk.decode_window_plan(L, 1, 1, 4, 16, -1)
    assert e.value.status == fk.ERR_INVALID_ARGUMENT
    s = fk.decode_window_plan(L, 1, 1, 4, 16, 64)
    assert s.splits <= 2
    # the splits cover the window's pages, not the whole table
    big = fk.cache_layout(8, 128, 4096)
    full = fk.decode_plan(big, 4, 32, 512, 0)
    win = fk.decode_window_plan(big, 4, 1, 32, 512, 256, 0)
    assert win.splits <= 6 < full.splits


def test_decode_with_options_host_checks():
    """fp4kv_decode_with_options refuses unknown option values, one of
    k_new / v_new alone, an append with several query tokens or a window,
    and kernels that do not serve the cache, before any HIP call."""
    L = fk.cache_layout(2, 128, 64)
    L8 = fk.cache_layout(2, 128, 64, format=fk.FORMAT_FP8_E4M3, k_scale=1.0, v_scale=1.0)
    L64 = fk.cache_layout(2, 64, 64)
    lib = fk.library()
    ok = 0x10000
    ws = fk.decode_window_plan(L, 2, 2, 8, 8, 0).workspace_bytes

    def call(layout=L, kn=None, vn=None, qt=1, window=0, kernel=0, merge=0, opts=True, min_len=0, out=ok):
        o = fk.DecodeOptions(kernel, merge, min_len)
        return lib.fp4kv_decode_with_options(ctypes.byref(layout), ok, kn, vn, ok, 2, qt, 8, ok, ok, 8, window,
                                             ctypes.c_float(0.1), 0, ok, ws, out,
                                             ctypes.byref(o) if opts else None, None)

    assert call(kernel=99) == fk.ERR_INVALID_ARGUMENT
    assert call(kernel=-1) == fk.ERR_INVALID_ARGUMENT
    assert call(merge=7) == fk.ERR_INVALID_ARGUMENT
    assert call(merge=3) == fk.ERR_INVALID_ARGUMENT
    assert call(min_len=-1) == fk.ERR_INVALID_ARGUMENT
    assert call(out=None) == fk.ERR_INVALID_ARGUMENT              # out is needed unless the merge is none
    assert call(merge=2, out=None, kernel=99) == fk.ERR_INVALID_ARGUMENT
    assert call(out=ok + 4) == fk.ERR_MISALIGNED
    assert call(kn=ok) == fk.ERR_INVALID_ARGUMENT                 # v_new missing
    assert call(kn=ok, vn=ok, qt=2) == fk.ERR_UNSUPPORTED
    assert call(kn=ok, vn=ok, window=64) == fk.ERR_UNSUPPORTED
    assert call(kernel=3, qt=2) == fk.ERR_UNSUPPORTED             # vector-ALU kernel: one query token
    assert call(kernel=3, window=64) == fk.ERR_UNSUPPORTED        # ... and no window
    assert call(layout=L8, kernel=2) == fk.ERR_UNSUPPORTED        # FP8 has its own kernel only
    assert call(layout=L64, kernel=1) == fk.ERR_UNSUPPORTED       # staged kernel: D = 128
    assert call(kn=ok + 8, vn=ok) == fk.ERR_MISALIGNED
