"""GPU-side set-up shared by the tests, the smoke check and the benchmark.

Builds a quantised cache for a workload of fp4kv_workloads (generating the
bf16 K/V rows on the CPU in seeded chunks, copying them to the device and
appending them with the library), and reads cache pages back in token-major
order for comparison with the oracle.  Only the library's entry points touch
the data on the device.
"""
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_workloads as wl

APPEND_CHUNK = 16384            # tokens per quantize_append call while filling a cache


@dataclass
class GpuCache:
    workload: wl.Workload
    layout: fk.CacheLayout
    cache: torch.Tensor                   # uint8 [cache_bytes] on the device
    page_table: torch.Tensor              # int32 [B][max_pages] on the device
    seq_lens: torch.Tensor                # int32 [B] on the device
    pt_cpu: wl.PageTable
    lens_cpu: torch.Tensor                # int64 [B]
    kept: Dict[int, tuple] = field(default_factory=dict)   # seq -> (k, v) bf16 CPU rows


def _append_rows(layout, cache, k, v, slots, device):
    kd = k.to(device, non_blocking=False)
    vd = v.to(device, non_blocking=False)
    sd = slots.to(device)
    fk.quantize_append(layout, kd, vd, sd, cache)


def build_cache(w: wl.Workload, seed: int, device="cuda", keep_seqs=(), extra_tokens=0,
                seqs: Optional[List[int]] = None, zero=True, fmt: str = "fp4") -> GpuCache:
    """Quantise every sequence's context into a fresh cache.

    Contiguous workloads get an identity page table; the paged workload gets
    seeded lengths and a seeded random page table with room for
    `extra_tokens` more tokens per sequence.  `seqs` limits which sequences
    are filled (others stay zero); `keep_seqs` keeps their bf16 rows on the
    CPU for the oracle.  fmt "fp8" builds an FP8 E4M3 cache with the
    workload's per-tensor scales, "fp8t" one with per-token scales."""
    lens = wl.seq_lengths(w, seed)
    if w.kind == "paged":
        pt = wl.random_page_table(lens, extra_tokens, seed, w.name)
    else:
        pt = wl.identity_page_table(w.batch, int(lens.max()) + extra_tokens)
    if fmt == "fp8":
        ks, vs = wl.fp8_tensor_scales(w, seed)
        layout = fk.cache_layout(w.kv_heads, w.head_dim, pt.num_pages, format=fk.FORMAT_FP8_E4M3,
                                 k_scale=ks, v_scale=vs)
    elif fmt == "fp8t":
        layout = fk.cache_layout(w.kv_heads, w.head_dim, pt.num_pages, format=fk.FORMAT_FP8_E4M3_TOKEN)
    else:
        layout = fk.cache_layout(w.kv_heads, w.head_dim, pt.num_pages)
    cache = (torch.zeros if zero else torch.empty)(layout.cache_bytes, dtype=torch.uint8, device=device)
    fk_k = wl.channel_factors(w, seed, "k")
    fk_v = wl.channel_factors(w, seed, "v")
    kept = {}
    for b in (range(w.batch) if seqs is None else seqs):
        L = int(lens[b])
        ks, vs = [], []
        for t0 in range(0, L, APPEND_CHUNK):
            t1 = min(L, t0 + APPEND_CHUNK)
            k = wl.kv_tokens(w, seed, b, "k", t0, t1, fk_k)
            v = wl.kv_tokens(w, seed, b, "v", t0, t1, fk_v)
            _append_rows(layout, cache, k, v, wl.slots_for(pt.table, b, t0, t1), device)
            if b in keep_seqs:
                ks.append(k)
                vs.append(v)
        if b in keep_seqs:
            kept[b] = (torch.cat(ks) if ks else torch.empty(0, w.kv_heads, w.head_dim, dtype=torch.bfloat16),
                       torch.cat(vs) if vs else torch.empty(0, w.kv_heads, w.head_dim, dtype=torch.bfloat16))
    torch.cuda.synchronize()
    return GpuCache(w, layout, cache, pt.table.to(device), lens.to(torch.int32).to(device),
                    pt, lens, kept)


def _v_token_major(codes_plane: np.ndarray, scales_plane: np.ndarray, D: int):
    """V planes of pages [P][H][...] in the stored order -> token-major
    (code bytes [P][H][64][D/2] with channel 2i in the low nibble, scales
    [P][H][64][D/16]).  Stored: codes row (slice, channel) of 8 bytes, two
    tokens per byte (even token low); scales row (slice, block) of 16."""
    P, H = codes_plane.shape[:2]
    c = codes_plane.reshape(P, H, 4, D, 8)                          # slice, channel, byte
    nib = np.stack([c & 0xF, c >> 4], axis=-1).reshape(P, H, 4, D, 16)   # slice, channel, token-in-slice
    nib = nib.transpose(0, 1, 2, 4, 3).reshape(P, H, 64, D)          # token, channel
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    s = scales_plane.reshape(P, H, 4, D // 16, 16).transpose(0, 1, 2, 4, 3).reshape(P, H, 64, D // 16)
    return packed, s


def read_pages(cache: torch.Tensor, layout: fk.CacheLayout, pages, n_tokens: int):
    """Stored bytes of the first n_tokens slots of a list of pages (all KV
    heads), token-major: K code bytes [n][H][D/2], K scales [n][H][D/16], V
    code bytes [n][H][D/2], V scales [n][H][D/16] (two codes per byte,
    channel 2i in the low nibble).  Only those pages are copied off the
    device."""
    H, D = layout.num_kv_heads, layout.head_dim
    idx = torch.as_tensor(np.asarray(pages, np.int64), device=cache.device)
    blocks = cache[: layout.cache_bytes].view(-1, H, layout.block_bytes)[idx].cpu().numpy()
    P = len(pages)

    def plane(off, size):
        return blocks[:, :, off:off + size]

    kc = plane(layout.k_codes_offset, 64 * D // 2).reshape(P, H, 64, D // 2)
    ks = plane(layout.k_scales_offset, 64 * D // 16).reshape(P, H, 64, D // 16)
    vc, vs = _v_token_major(plane(layout.v_codes_offset, 64 * D // 2),
                            plane(layout.v_scales_offset, 64 * D // 16), D)

    def tok(x):
        return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(P * 64, H, x.shape[-1])[:n_tokens])

    return tok(kc), tok(ks), tok(vc), tok(vs)


def read_pages_fp8(cache: torch.Tensor, layout: fk.CacheLayout, pages, n_tokens: int):
    """Stored codes of the first n_tokens slots of a list of pages of an FP8
    cache, token-major: K [n][H][D], V [n][H][D] (V un-laid from its
    [slice][half][channel][8 tokens] rows)."""
    H, D = layout.num_kv_heads, layout.head_dim
    idx = torch.as_tensor(np.asarray(pages, np.int64), device=cache.device)
    blocks = cache[: layout.cache_bytes].view(-1, H, layout.block_bytes)[idx].cpu().numpy()
    P = len(pages)
    kc = blocks[:, :, layout.k_codes_offset:layout.k_codes_offset + 64 * D].reshape(P, H, 64, D)
    v = blocks[:, :, layout.v_codes_offset:layout.v_codes_offset + 64 * D].reshape(P, H, 4, 2, D, 8)
    vc = v.transpose(0, 1, 2, 3, 5, 4).reshape(P, H, 64, D)         # token = 16*slice + 8*half + i

    def tok(x):
        return np.ascontiguousarray(x.transpose(0, 2, 1, 3).reshape(P * 64, H, D)[:n_tokens])

    return tok(kc), tok(vc)


def read_token_scales(cache: torch.Tensor, layout: fk.CacheLayout, pages, n_tokens: int):
    """fp16 scale patterns of the first n_tokens slots of a list of pages of
    an FP8 cache with per-token scales, token-major: K [n][H], V [n][H]."""
    H = layout.num_kv_heads
    idx = torch.as_tensor(np.asarray(pages, np.int64), device=cache.device)
    blocks = cache[: layout.cache_bytes].view(-1, H, layout.block_bytes)[idx].cpu().numpy()
    P = len(pages)

    def plane(off):
        s = np.ascontiguousarray(blocks[:, :, off:off + 128]).view(np.uint16).reshape(P, H, 64)
        return np.ascontiguousarray(s.transpose(0, 2, 1).reshape(P * 64, H)[:n_tokens])

    return plane(layout.k_scales_offset), plane(layout.v_scales_offset)


def row_rel_error(out: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output row (last axis): max |out - ref| / max |ref| (0 where both
    rows are zero)."""
    num = np.max(np.abs(out.astype(np.float64) - ref), axis=-1)
    den = np.max(np.abs(ref), axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def unpack_int_codes(codes, bits: int, head_dim: int) -> np.ndarray:
    """Integer-format code bytes [B][H][T][D * bits / 8] (device or host) ->
    signed codes int8 [B][T][H][D], token-major like the input rows.  Within
    a row, channel i sits in bits bits*(i % (8/bits)) .. of byte i*bits/8,
    two's complement."""
    c = codes.cpu().numpy() if hasattr(codes, "cpu") else np.asarray(codes)
    B, H, T, _ = c.shape
    if bits == 8:
        v = c.view(np.int8).astype(np.int8)
    else:
        per = 8 // bits
        shifts = (np.arange(per) * bits).astype(np.uint8)
        f = (c[..., None] >> shifts) & ((1 << bits) - 1)                # [B][H][T][R][per]
        f = f.reshape(B, H, T, head_dim).astype(np.int16)
        v = np.where(f >= (1 << (bits - 1)), f - (1 << bits), f).astype(np.int8)
    return np.ascontiguousarray(v.reshape(B, H, T, head_dim).transpose(0, 2, 1, 3))


def int_scales_host(scales, granularity: str) -> np.ndarray:
    """Device fp16 scale patterns -> uint16, per token [B][T][H] (from
    [B][H][T]) or per channel [B][H][D] (as stored)."""
    s = scales.cpu().numpy().view(np.uint16)
    return np.ascontiguousarray(s.transpose(0, 2, 1)) if granularity == "token" else s
