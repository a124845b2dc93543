"""Pins for the oracle's integer formats of the bit-width sweep (CPU only).

"Quantising the KV cache", Concept section, results table: INT8 / INT4 / INT2
with one scale per token, and with K per channel and V per token; Maths
section: one FP16 scale per group.  The page prints no integer encoder; the
oracle reads it as symmetric (qmax = 2^(b-1) - 1), scale = fp16 nearest-even
of amax / qmax (a zero scale becoming the smallest fp16 subnormal), codes =
nearest-even integer of x / scale capped at qmax.  These tests check that rule
with independent means: numpy's float16 conversion and rint (library
rounding), exact Fractions, transposition, and closed forms.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import exact_checker as ex
import fp4kv_workloads as wl

ALL_POS = np.array([b for b in range(1, 0x7F80)], np.uint16)        # positive finite bf16
QMAX = {8: 127, 4: 7, 2: 1}


def _bf16(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _np_scale_code(amax, qmax):
    """Library statement of the scale rule: numpy rounds the float64 quotient
    to float16 to nearest even.  The float64 quotient of a bf16 value by a
    7-bit integer is either exactly an fp16 rounding midpoint or at least
    2^-27 (relative) away from every one, so rounding it first changes
    nothing."""
    with np.errstate(over="ignore"):
        h = (amax / qmax).astype(np.float16)
    code = h.view(np.uint16).astype(np.int64)
    code = np.where(np.isinf(h), 0x7BFF, code)
    return np.where(code == 0, 1, code)


def test_fp16_table_matches_library(oracle_mod):
    ref = np.arange(0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    assert np.array_equal(oracle_mod.fp16_table(), ref)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_scale_rule_every_bf16_amax(oracle_mod, bits):
    """Groups of one element: every positive finite bf16 as amax."""
    x = ALL_POS.reshape(-1, 1, 1)
    codes, scales = oracle_mod.quantize_int(x, bits, "token")
    want = _np_scale_code(_bf16(ALL_POS), QMAX[bits])
    assert np.array_equal(scales[:, 0].astype(np.int64), want)
    # saturation and the subnormal fallback both occur in this sweep
    assert (scales == 0x7BFF).any() and (scales == 1).any()
    # a lone element maps to qmax when its scale is a normal, unsaturated
    # fp16 (then amax / s is within qmax * 2^-11 of qmax)
    s = scales[:, 0].view(np.float16).astype(np.float64)
    normal = (scales[:, 0] != 0x7BFF) & (scales[:, 0] >= 0x0400)
    assert np.all(codes[normal, 0, 0] == QMAX[bits])
    # the fallback: a scale of 2^-24 and the nearest code to x / 2^-24
    fb = scales[:, 0] == 1
    assert np.array_equal(codes[fb, 0, 0], np.minimum(np.rint(_bf16(ALL_POS[fb]) / s[fb]), QMAX[bits]))


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4123, 0x3C01, 0x0400, 0x4B7F, 0x2F55])
def test_element_rule_every_bf16_value(oracle_mod, bits, amax_bits):
    """Groups of [amax, x] for every bf16 magnitude x <= amax and its negation:
    the code of x against numpy rint (nearest even) of the float64 quotient,
    capped at qmax, with the sign of x."""
    amax = _bf16(np.array([amax_bits], np.uint16))[0]
    mags = ALL_POS[_bf16(ALL_POS) <= amax]
    mags = np.concatenate([[0], mags]).astype(np.uint16)
    for sign in (0, 0x8000):
        x = np.stack([np.full(mags.size, amax_bits, np.uint16), mags | sign], axis=1).reshape(-1, 1, 2)
        codes, scales = oracle_mod.quantize_int(x, bits, "token")
        s = scales[:, 0].view(np.float16).astype(np.float64)
        want = np.minimum(np.rint(_bf16(mags) / s), QMAX[bits]).astype(np.int64)
        if sign:
            want = -want
        assert np.array_equal(codes[:, 0, 1].astype(np.int64), want)


def test_ties_go_to_the_even_integer(oracle_mod):
    """x = (k + 1/2) * s exactly: the code is whichever of k, k + 1 is even."""
    s_bits = 0x3C00                                   # fp16 1.0
    qmax = 127
    for k in range(0, 126):
        amax = np.float32(qmax)                      # amax / qmax = 1.0 exactly
        xv = np.float32(k + 0.5)
        x = np.array([amax, xv, -xv], np.float32).view(np.uint32) >> 16
        codes, scales = oracle_mod.quantize_int(x.astype(np.uint16).reshape(1, 1, 3), 8, "token")
        assert scales[0, 0] == s_bits
        even = k if k % 2 == 0 else k + 1
        assert codes[0, 0].tolist() == [qmax, even, -even]


def test_brute_force_fractions(oracle_mod):
    """Groups of 3 over a small value set, each code and scale from exact
    Fractions by a nearest-entry search (fp16 table from numpy's decoder)."""
    fp16 = [Fraction(float(v)) for v in np.arange(0x7C00, dtype=np.uint16).view(np.float16)]
    vals = [0x0000, 0x3F80, 0xBFC0, 0x4040, 0x3E2B, 0xC2F0, 0x3A01, 0x0080, 0x4780]
    rng = np.random.default_rng(3)
    groups = rng.choice(np.array(vals, np.uint16), size=(300, 3))
    for bits in (8, 4, 2):
        qmax = QMAX[bits]
        codes, scales = oracle_mod.quantize_int(groups.reshape(300, 1, 3), bits, "token")
        for i, grp in enumerate(groups.tolist()):
            fr = [ex.bf16_fraction(b) for b in grp]
            sc = ex.nearest_code_sorted(max(abs(v) for v in fr) / qmax, fp16) or 1
            assert scales[i, 0] == sc
            s = fp16[sc]
            for j, v in enumerate(fr):
                y = abs(v) / s
                k = int(y)                           # floor
                c = k + 1 if (y - k > Fraction(1, 2) or (y - k == Fraction(1, 2) and k % 2)) else k
                c = min(c, qmax)
                assert codes[i, 0, j] == (-c if v < 0 else c), (bits, grp, j)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_round_trip_of_representable_values(oracle_mod, bits):
    """Integers in [-qmax, qmax] times a power of two, with qmax present:
    quantised back to the same integers, scale exactly the power of two."""
    qmax = QMAX[bits]
    rng = np.random.default_rng(bits)
    for e in (-6, 0, 3):
        ints = rng.integers(-qmax, qmax + 1, size=(40, 2, 16))
        ints[:, :, 0] = qmax
        x = torch.tensor(ints * 2.0 ** e, dtype=torch.float32).to(torch.bfloat16)
        codes, scales = oracle_mod.quantize_int(x, bits, "token")
        assert np.array_equal(codes, ints)
        assert np.all(scales.view(np.float16).astype(np.float64) == 2.0 ** e)
        assert np.array_equal(oracle_mod.dequantize_int(codes, scales, "token"), ints * 2.0 ** e)


def test_int2_levels(oracle_mod):
    g = torch.Generator().manual_seed(9)
    x = torch.randn(64, 2, 32, generator=g).to(torch.bfloat16)
    codes, scales = oracle_mod.quantize_int(x, 2, "token")
    assert set(np.unique(codes).tolist()) == {-1, 0, 1}
    # the largest magnitude of each group maps to +-1
    a = np.abs(x.float().numpy())
    top = np.argmax(a, axis=-1)
    assert np.all(np.abs(np.take_along_axis(codes, top[..., None], -1)) == 1)


@pytest.mark.parametrize("bits", [8, 4])
def test_per_channel_is_per_token_of_the_transpose(oracle_mod, bits):
    """One channel of one head across the tokens is a group: the same codes
    and scales as per-token quantisation of the transposed rows."""
    g = torch.Generator().manual_seed(4)
    T, H, D = 37, 3, 16
    x = (torch.randn(T, H, D, generator=g) * torch.linspace(0.1, 9.0, D)).to(torch.bfloat16)
    c_ch, s_ch = oracle_mod.quantize_int(x, bits, "channel")
    xt = x.permute(2, 1, 0).contiguous()             # [D][H][T]: row = (channel, head) over tokens
    c_t, s_t = oracle_mod.quantize_int(xt, bits, "token")
    assert np.array_equal(c_ch, c_t.transpose(2, 1, 0))
    assert np.array_equal(s_ch, s_t.T)
    assert s_ch.shape == (H, D)


def test_rejects_bad_arguments(oracle_mod):
    x = np.array([[[0x3F80]]], np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.quantize_int(x, 1, "token")
    with pytest.raises(ValueError):
        oracle_mod.quantize_int(x, 4, "block")
    with pytest.raises(ValueError):
        oracle_mod.quantize_int(np.array([[[0x7F80]]], np.uint16), 4, "token")


def _q(G, D, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(G, D, generator=g).to(torch.bfloat16)


def test_attention_values_matches_library_sdpa(oracle_mod):
    g = torch.Generator().manual_seed(21)
    k = torch.randn(150, 64, generator=g, dtype=torch.float64) * 2
    v = torch.randn(150, 64, generator=g, dtype=torch.float64)
    q = _q(4, 64, 22)
    out = oracle_mod.attention_values(q, k.numpy(), v.numpy(), 0.125)
    qf = q.float().double()
    ref = F.scaled_dot_product_attention(qf[None], k[None], v[None], scale=0.125)[0].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


def test_attention_values_special_cases(oracle_mod):
    q = _q(3, 32, 5)
    v = np.random.default_rng(1).standard_normal((9, 32))
    one = oracle_mod.attention_values(q, np.ones((1, 32)), v[:1], 0.3)
    assert np.array_equal(one, np.repeat(v[:1], 3, 0))
    same = oracle_mod.attention_values(q, np.ones((9, 32)), v, 0.3)
    np.testing.assert_allclose(same, np.repeat(v.mean(0, keepdims=True), 3, 0), rtol=1e-13, atol=1e-15)
    empty = oracle_mod.attention_values(q, v[:0], v[:0], 0.3)
    assert not empty.any()


def test_decode_values_matches_single_problems(oracle_mod):
    rng = np.random.default_rng(8)
    lens = [0, 3, 70]
    kv = [rng.standard_normal((max(n, 1), 2, 16)) for n in lens]
    vv = [rng.standard_normal((max(n, 1), 2, 16)) for n in lens]
    q = torch.randn(3, 6, 16, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    out = oracle_mod.decode_attention_values(q, kv, vv, lens, 0.25)
    for b, n in enumerate(lens):
        for h in range(2):
            ref = oracle_mod.attention_values(q[b, 3 * h:3 * h + 3], kv[b][:n, h], vv[b][:n, h], 0.25)
            assert np.array_equal(out[b, 3 * h:3 * h + 3], ref)


def test_per_channel_keys_beat_per_token_on_outlier_channels(oracle_mod):
    """The page's KIVI remark: keys with a few fixed large channels are better
    quantised per channel.  On the 4-KV-head workload's keys (four channels
    per head x10) INT4 per channel has a smaller error than INT4 per token;
    and the error falls as bits rise."""
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    k = wl.kv_tokens(w, 2, 0, "k", 0, 512)
    exact = oracle_mod.bf16_values(k)
    err = {}
    for bits in (8, 4, 2):
        for gran in ("token", "channel"):
            c, s = oracle_mod.quantize_int(k, bits, gran)
            err[bits, gran] = np.sqrt(np.mean((oracle_mod.dequantize_int(c, s, gran) - exact) ** 2))
    assert err[4, "channel"] < 0.5 * err[4, "token"]
    for gran in ("token", "channel"):
        assert err[8, gran] < err[4, gran] < err[2, gran]
