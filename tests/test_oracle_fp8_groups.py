"""Pins for the oracle's FP8 E4M3 formats with an fp16 scale per token or per
channel (CPU only).

"KV Cache Quantisation", Common questions: when checking quality, sweep the
FP8 scale granularities as well as FP16 and the FP4 layouts.  "Quantising the
KV cache", Concept section: a per-token scale covers one token's channels, a
per-channel scale one channel across the tokens.  The pages print no encoder
for these; the oracle reads it as the page's FP4 encoder with E4M3 elements
and the integer rows' fp16 scale: scale = fp16 nearest-even of amax / 448
(zero becoming the smallest fp16 subnormal), code = sign | E4M3 nearest-even,
saturating, of |x| / scale.  These tests check that rule by independent means:
numpy's float16 and torch's float8_e4m3fn conversions (library rounding),
exact Fractions, closed forms and transposition.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import exact_checker as ex

ALL_POS = np.array([b for b in range(1, 0x7F80)], np.uint16)        # positive finite bf16


def _bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _np_scale_code(amax):
    """Library statement of the scale rule: numpy rounds the float64 quotient
    amax / 448 to float16, nearest even.  A bf16 value (8 significant bits)
    over 448 = 7 * 2^6 is either exactly an fp16 rounding midpoint (12 bits,
    times 448: 15 bits) or at least 2^-16 (relative) away from every one, so
    rounding to float64 first changes nothing."""
    with np.errstate(over="ignore"):
        h = (amax / 448.0).astype(np.float16)
    code = h.view(np.uint16).astype(np.int64)
    code = np.where(np.isinf(h), 0x7BFF, code)
    return np.where(code == 0, 1, code)


def _torch_e4m3_codes(y32):
    """torch's float8_e4m3fn codes (nearest even) of fp32 magnitudes below
    464, where torch's conversion does not overflow."""
    t = torch.from_numpy(np.ascontiguousarray(y32, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().astype(np.int64)


def test_scale_rule_every_bf16_amax(oracle_mod):
    """Groups of one element: every positive finite bf16 as amax."""
    x = ALL_POS.reshape(-1, 1, 1)
    codes, scales = oracle_mod.quantize_fp8_groups(x, "token")
    assert np.array_equal(scales[:, 0].astype(np.int64), _np_scale_code(_bf16(ALL_POS)))
    # saturation and the subnormal fallback both occur in this sweep
    assert (scales == 0x7BFF).any() and (scales == 1).any()
    # a lone element maps to 448 (code 0x7E) when its scale is a normal,
    # unsaturated fp16: amax / s is within 448 * 2^-11 of 448
    normal = (scales[:, 0] != 0x7BFF) & (scales[:, 0] >= 0x0400)
    assert np.all(codes[normal, 0, 0] == 0x7E)
    # with the smallest scale 2^-24 (the fallback, or amax / 448 rounding to
    # it) the code is torch's E4M3 of x * 2^24, saturated at 448
    fb = scales[:, 0] == 1
    want = _torch_e4m3_codes(np.minimum(_bf16(ALL_POS[fb]) * 2.0 ** 24, 448.0).astype(np.float32))
    assert np.array_equal(codes[fb, 0, 0].astype(np.int64), want)


@pytest.mark.parametrize("amax_bits", [0x43E0, 0x3F80, 0x4123, 0x3C01, 0x0400, 0x4B7F, 0x2F55])
def test_element_rule_every_bf16_value(oracle_mod, amax_bits):
    """Groups of [amax, x] for every bf16 magnitude x <= amax and its negation:
    the code of x against torch's float8_e4m3fn conversion of the fp32
    quotient x / s, with the sign of x in bit 7.  A bf16 x over an fp16 s is
    either exactly an E4M3 rounding midpoint (5 significant bits) or at least
    2^-17 (relative) away from every one, so the correctly rounded fp32
    quotient rounds like the exact one."""
    amax = _bf16(np.array([amax_bits], np.uint16))[0]
    mags = ALL_POS[_bf16(ALL_POS) <= amax]
    mags = np.concatenate([[0], mags]).astype(np.uint16)
    for sign in (0, 0x8000):
        x = np.stack([np.full(mags.size, amax_bits, np.uint16), mags | sign], axis=1).reshape(-1, 1, 2)
        codes, scales = oracle_mod.quantize_fp8_groups(x, "token")
        assert np.all(scales == scales[0, 0])
        s = np.float32(scales[0, 0].view(np.float16))
        want = _torch_e4m3_codes(_bf16(mags).astype(np.float32) / s)
        if sign:
            want = want | 0x80
        assert np.array_equal(codes[:, 0, 1].astype(np.int64), want)


def test_ties_go_to_the_even_code(oracle_mod):
    """x exactly halfway between two E4M3 magnitudes (scale 1: amax 448):
    the code is whichever neighbour is even."""
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for k in range(0, 126):
        mid = (e4[k] + e4[k + 1]) / 2                 # 5 significant bits: exact in bf16
        x = np.array([448.0, mid, -mid], np.float32).view(np.uint32) >> 16
        codes, scales = oracle_mod.quantize_fp8_groups(x.astype(np.uint16).reshape(1, 1, 3), "token")
        assert scales[0, 0] == 0x3C00                 # fp16 1.0
        even = k if k % 2 == 0 else k + 1
        assert codes[0, 0].tolist() == [0x7E, even, 0x80 | even]


def test_brute_force_fractions(oracle_mod):
    """Groups of 3 over a small value set: each scale and code from exact
    Fractions by a nearest-entry search (fp16 table from numpy's decoder,
    E4M3 table from torch's)."""
    fp16 = [Fraction(float(v)) for v in np.arange(0x7C00, dtype=np.uint16).view(np.float16)]
    vals = [0x0000, 0x3F80, 0xBFC0, 0x4040, 0x3E2B, 0xC2F0, 0x3A01, 0x0080, 0x4780, 0x43E0, 0x8000]
    rng = np.random.default_rng(5)
    groups = rng.choice(np.array(vals, np.uint16), size=(300, 3))
    codes, scales = oracle_mod.quantize_fp8_groups(groups.reshape(300, 1, 3), "token")
    for i, grp in enumerate(groups.tolist()):
        fr = [ex.bf16_fraction(b) for b in grp]
        sc = ex.nearest_code_sorted(max(abs(v) for v in fr) / 448, fp16) or 1
        assert scales[i, 0] == sc
        s = fp16[sc]
        for j, (b, v) in enumerate(zip(grp, fr)):
            c = ex.nearest_code_sorted(abs(v) / s, ex.E4M3)
            assert codes[i, 0, j] == (c | (0x80 if b & 0x8000 else 0)), (grp, j)


def test_round_trip_of_representable_values(oracle_mod):
    """E4M3 magnitudes times a scale of at most 4 significant bits, with 448
    present: the same codes back, the scale exactly, the values exactly."""
    rng = np.random.default_rng(8)
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for s in (2.0 ** -10, 0.75, 1.0, 1.5 * 2.0 ** 4, 13 * 2.0 ** -3):
        c = rng.integers(0, 127, size=(30, 2, 16))
        c[:, :, 0] = 126
        neg = rng.integers(0, 2, size=c.shape)
        vals = np.where(neg == 1, -e4[c], e4[c]) * s
        x = torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16)
        assert np.array_equal(x.double().numpy(), vals)            # exactly representable
        codes, scales = oracle_mod.quantize_fp8_groups(x, "token")
        assert np.all(scales.view(np.float16).astype(np.float64) == s)
        want = c | np.where(neg == 1, 0x80, 0)
        # a zero magnitude keeps its sign only when the input is -0.0: torch
        # makes -0.0 of a negative zero product, so the sign bit survives
        assert np.array_equal(codes.astype(np.int64), want)
        assert np.array_equal(oracle_mod.dequantize_fp8_groups(codes, scales, "token"), vals)


def test_dequantize_matches_library(oracle_mod):
    """+-E4M3(code) * fp16(scale) against torch's float8_e4m3fn decoder."""
    g = torch.Generator().manual_seed(6)
    x = (torch.randn(50, 3, 64, generator=g) * 3).to(torch.bfloat16)
    for gran in ("token", "channel"):
        codes, scales = oracle_mod.quantize_fp8_groups(x, gran)
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        s = scales.view(np.float16).astype(np.float64)
        want = v * (s[..., None] if gran == "token" else s[None])
        assert np.array_equal(oracle_mod.dequantize_fp8_groups(codes, scales, gran), want)
        # error at most half an E4M3 step: 2^-4 relative for normal codes
        err = np.abs(oracle_mod.dequantize_fp8_groups(codes, scales, gran) - x.double().numpy())
        assert np.all(err <= np.abs(x.double().numpy()) * 2.0 ** -4 + (s.max() * 2.0 ** -10))


def test_per_channel_is_per_token_of_the_transpose(oracle_mod):
    """One channel of one head across the tokens is a group: the same codes
    and scales as per-token quantisation of the transposed rows."""
    g = torch.Generator().manual_seed(4)
    T, H, D = 37, 3, 16
    x = (torch.randn(T, H, D, generator=g) * torch.linspace(0.1, 9.0, D)).to(torch.bfloat16)
    c_ch, s_ch = oracle_mod.quantize_fp8_groups(x, "channel")
    c_t, s_t = oracle_mod.quantize_fp8_groups(x.permute(2, 1, 0).contiguous(), "token")
    assert np.array_equal(c_ch, c_t.transpose(2, 1, 0))
    assert np.array_equal(s_ch, s_t.T)
    assert s_ch.shape == (H, D)


def test_saturated_scale(oracle_mod):
    """amax / 448 above 65504: the scale saturates at 65504 and every
    quotient at or above 448 saturates to code 0x7E."""
    big = np.array([0x7F00, 0x7E00, 0x4780, 0xFF00], np.uint16).reshape(1, 1, 4)   # 1.7e38, 4.3e37, 65536, -1.7e38
    codes, scales = oracle_mod.quantize_fp8_groups(big, "token")
    assert scales[0, 0] == 0x7BFF
    assert codes[0, 0, 0] == 0x7E and codes[0, 0, 1] == 0x7E and codes[0, 0, 3] == 0xFE
    assert codes[0, 0, 2] == _torch_e4m3_codes(np.array([65536.0 / 65504.0], np.float32))[0]


def test_rejects_bad_input(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.quantize_fp8_groups(np.array([[[0x7F80]]], np.uint16), "token")
    with pytest.raises(ValueError):
        oracle_mod.quantize_fp8_groups(np.array([[[0x3F80]]], np.uint16), "block")
