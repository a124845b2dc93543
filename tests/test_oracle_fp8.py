"""Pins for the oracle's FP8 E4M3 variant with one scale per tensor (CPU only).

"Quantising the KV cache", Concept section, results table: FP8 E4M3 with one
scale per tensor, 8 bits per number.  The rounding follows the page's encoder
(nearest, ties to the even code, saturating), applied to x / scale.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import exact_checker as ex

ALL_FINITE = np.array([b for b in range(0x10000) if (b >> 7) & 0xFF != 0xFF], np.uint16)


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -4, 2.0 ** 5, 2.0 ** -10])
def test_every_bf16_vs_library_fp8_power_of_two_scales(oracle_mod, scale):
    """With a power-of-two scale x / scale is exact in fp32, so torch's
    float8_e4m3fn conversion (nearest even) is an independent statement of the
    rule wherever it does not overflow; past 464 it gives NaN where the
    format here saturates to 448."""
    codes = oracle_mod.quantize_fp8(ALL_FINITE, scale)
    y = torch.from_numpy(_bf16_value(ALL_FINITE)) / scale
    ref = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    nan = (ref & 0x7F) == 0x7F
    assert np.array_equal(codes[~nan], ref[~nan])
    assert nan.any() and (~nan).sum() > 30000
    assert np.all((codes[nan] & 0x7F) == 126)
    assert np.array_equal(codes[nan] >> 7, ref[nan] >> 7)


@pytest.mark.parametrize("scale", [0.75, 0.0173, 3.3, 1.0 / 7.0, 123.456])
def test_general_scales_vs_exact_rational(oracle_mod, scale):
    """Any fp32 scale: nearest-even rounding of the exact quotient, checked by
    the Fraction-based nearest-code search (a different algorithm) on every
    bf16 magnitude whose quotient lies in the E4M3 range, plus saturation.
    Scale 0.75 puts many quotients exactly on rounding midpoints."""
    s32 = float(np.float32(scale))
    mags = ALL_FINITE[ALL_FINITE < 0x8000]
    codes = oracle_mod.quantize_fp8(mags, s32)
    s = Fraction(s32)
    ties = 0
    for bits, code in zip(mags.tolist(), codes.tolist()):
        y = ex.bf16_fraction(bits) / s
        want = ex.nearest_code_sorted(y, ex.E4M3)
        assert code == want, (hex(bits), code, want)
        if y < ex.E4M3[-1] and want + 1 < len(ex.E4M3) and 2 * y == ex.E4M3[want] + ex.E4M3[want + 1]:
            ties += 1
    if scale == 0.75:
        assert ties > 30


def test_sign_kept_and_zero(oracle_mod):
    x = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x3F80, 0xBF80], np.uint16)   # 0, -0, tiny, -tiny, 1, -1
    c = oracle_mod.quantize_fp8(x, 1.0)
    assert c.tolist() == [0x00, 0x80, 0x00, 0x80, 0x38, 0xB8]
    mags = ALL_FINITE[ALL_FINITE < 0x8000]
    assert np.array_equal(oracle_mod.quantize_fp8(mags | 0x8000, 0.3), oracle_mod.quantize_fp8(mags, 0.3) | 0x80)


def test_round_trip_of_representable_values(oracle_mod):
    """Every E4M3 value times a power-of-two scale is stored exactly."""
    table = oracle_mod.e4m3_table()
    for scale in (1.0, 0.125, 16.0):
        vals = torch.tensor(table * scale, dtype=torch.float32).to(torch.bfloat16)
        bits = vals.view(torch.int16).numpy().view(np.uint16)
        codes = oracle_mod.quantize_fp8(bits, scale)
        assert codes.tolist() == list(range(127))
        assert np.array_equal(oracle_mod.dequantize_fp8(codes, scale), table * scale)


def test_monotone_and_saturating(oracle_mod):
    mags = ALL_FINITE[ALL_FINITE < 0x7F80]
    order = np.argsort(_bf16_value(mags), kind="stable")
    codes = oracle_mod.quantize_fp8(mags[order], 0.05)
    assert np.all(np.diff(codes.astype(int)) >= 0)
    assert codes[-1] == 126 and codes[0] == 0


def test_rejects_bad_scale_and_non_finite(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.quantize_fp8(np.array([0x3F80], np.uint16), 0.0)
    with pytest.raises(ValueError):
        oracle_mod.quantize_fp8(np.array([0x3F80], np.uint16), float("inf"))
    with pytest.raises(ValueError):
        oracle_mod.quantize_fp8(np.array([0x7F80], np.uint16), 1.0)


def _rand(T, D, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    k = (torch.randn(T, D, generator=g) * scale).to(torch.bfloat16)
    v = torch.randn(T, D, generator=g).to(torch.bfloat16)
    q = torch.randn(4, D, generator=g).to(torch.bfloat16)
    bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    return bits(q), bits(k), bits(v)


def test_attention_single_token_and_empty(oracle_mod):
    q, k, v = _rand(1, 128, 3)
    kc, vc = oracle_mod.quantize_fp8(k, 0.02), oracle_mod.quantize_fp8(v, 0.01)
    out = oracle_mod.attention_fp8(q, kc, vc, 0.02, 0.01, 128 ** -0.5)
    assert np.array_equal(out, np.repeat(oracle_mod.dequantize_fp8(vc, 0.01), 4, 0))
    empty = oracle_mod.attention_fp8(q, kc[:0], vc[:0], 0.02, 0.01, 0.1)
    assert np.array_equal(empty, np.zeros_like(empty))


@pytest.mark.parametrize("T,kscale", [(7, 1.0), (300, 4.0)])
def test_attention_matches_library_sdpa(oracle_mod, T, kscale):
    """The fp64 definition against torch's scaled_dot_product_attention in
    float64 on the dequantised K and V."""
    q, k, v = _rand(T, 128, 10 + T, kscale)
    ks, vs = 0.05 * kscale, 0.01
    kc, vc = oracle_mod.quantize_fp8(k, ks), oracle_mod.quantize_fp8(v, vs)
    out = oracle_mod.attention_fp8(q, kc, vc, ks, vs, 0.09)
    qf = torch.from_numpy((q.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    kf = torch.from_numpy(oracle_mod.dequantize_fp8(kc, ks))
    vf = torch.from_numpy(oracle_mod.dequantize_fp8(vc, vs))
    ref = F.scaled_dot_product_attention(qf[None], kf[None], vf[None], scale=0.09)[0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_batch_matches_single_problems(oracle_mod):
    """The threaded batch entry (GQA mapping, ragged lengths) against the
    single-problem entry."""
    g = torch.Generator().manual_seed(5)
    B, Hkv, G, D = 3, 2, 2, 128
    lens = [0, 5, 70]
    kc = [oracle_mod.quantize_fp8((torch.randn(max(l, 1), Hkv, D, generator=g)).to(torch.bfloat16)
                                  .view(torch.int16).numpy().view(np.uint16), 0.03) for l in lens]
    vc = [oracle_mod.quantize_fp8((torch.randn(max(l, 1), Hkv, D, generator=g)).to(torch.bfloat16)
                                  .view(torch.int16).numpy().view(np.uint16), 0.02) for l in lens]
    q = torch.randn(B, Hkv * G, D, generator=g).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = oracle_mod.decode_attention_fp8(q, kc, vc, 0.03, 0.02, lens, 0.1)
    for b in range(B):
        for h in range(Hkv):
            ref = oracle_mod.attention_fp8(q[b, h * G:(h + 1) * G], kc[b][:lens[b], h], vc[b][:lens[b], h],
                                           0.03, 0.02, 0.1)
            assert np.array_equal(out[b, h * G:(h + 1) * G], ref)


def test_fp8_cost_from_the_page(oracle_mod):
    """Results table: FP8 with one scale per tensor is 8 bits per number, 50 %
    of FP16's memory."""
    assert oracle_mod.bits_per_number(8, 0, 0) == 8
    assert oracle_mod.fp8_cache_bytes(64, 1, 8, 128) == 64 * 2 * 8 * 128
    assert oracle_mod.fp8_cache_bytes(1, 1, 1, 128) / (2 * 128 * 2) == 0.5
