"""Pins for the oracle's FP4 quantiser (CPU only).

Each test checks the oracle against something other than itself: printed or
format-fixed tables, a library FP8 decoder/encoder, an exact-rational checker
written a different way (tests/exact_checker.py), a threshold-count rule, and
hand derivations of small blocks.
"""
from fractions import Fraction
import itertools

import numpy as np
import pytest
import torch

import exact_checker as ex


def all_bf16_magnitudes():
    """Every non-negative finite bf16 bit pattern: 0x0000 .. 0x7F7F."""
    return np.arange(0, 0x7F80, dtype=np.uint16)


def bf16_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ------------------------------------------------------------------ formats

def test_e2m1_table_matches_golden(oracle_mod):
    golden = [float(r[1]) for r in ex.read_table("e2m1_magnitudes.txt")]
    assert oracle_mod.e2m1_table().tolist() == golden
    # the page divides amax by 6, so 6 must be the largest element magnitude
    assert oracle_mod.e2m1_table().max() == 6.0


def test_e4m3_table_matches_library_decoder(oracle_mod):
    lib_vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    assert oracle_mod.e4m3_table().tolist() == lib_vals.tolist()


def test_e4m3_landmarks(oracle_mod):
    for code, val in ex.read_table("e4m3_landmarks.txt"):
        assert oracle_mod.e4m3_value(int(code, 16)) == float(val)


# --------------------------------------------------------------- scale rule

def test_scale_rule_exhaustive_vs_library_fp8(oracle_mod):
    """All 32,640 non-negative finite bf16 block maxima: the scale code equals
    torch's float8_e4m3fn rounding of amax/6, with the page's zero fallback
    and saturation (torch yields NaN past 464) applied on top."""
    a = all_bf16_magnitudes()
    _, sc, _ = oracle_mod.quantize(a.reshape(-1, 1), want_xhat=False)
    y = torch.from_numpy(bf16_to_f64(a)) / 6.0
    lib = y.to(torch.float8_e4m3fn).view(torch.uint8).to(torch.int64)
    lib = torch.where(y >= 464.0, torch.tensor(126), lib)       # saturate instead of NaN
    lib = torch.where(lib == 0, torch.tensor(1), lib)           # zero scale -> min subnormal
    assert np.array_equal(sc[:, 0].astype(np.int64), lib.numpy())


def test_scale_rule_exhaustive_vs_exact_rational(oracle_mod):
    a = all_bf16_magnitudes()
    _, sc, _ = oracle_mod.quantize(a.reshape(-1, 1), want_xhat=False)
    want = np.array([ex.scale_code(ex.bf16_fraction(int(b))) for b in a], np.uint8)
    assert np.array_equal(sc[:, 0], want)
    # the E4M3 ties (amax/6 exactly halfway between two codes) are covered
    ties = sum(1 for b in a if _is_e4m3_tie(ex.bf16_fraction(int(b)) / 6))
    assert ties > 100


def _is_e4m3_tie(y):
    for lo, hi in zip(ex.E4M3[:-1], ex.E4M3[1:]):
        if lo < y < hi:
            return y - lo == hi - y
    return False


# ------------------------------------------------------------- element rule

# thresholds t on q = |x|/s between consecutive E2M1 codes, and whether an
# exact tie moves up (the upper code is even)
_THRESHOLDS = [(0.25, False), (0.75, True), (1.25, False), (1.75, True),
               (2.5, False), (3.5, True), (5.0, False)]


import functools


@functools.lru_cache(maxsize=None)
def _largest_amax_per_scale():
    """For each scale code 1..126, the largest bf16 block maximum giving it
    (found with the exact checker)."""
    best = {}
    for b in all_bf16_magnitudes()[1:]:
        sc = ex.scale_code(ex.bf16_fraction(int(b)))
        best[sc] = int(b)
    return best


def test_element_rule_exhaustive_threshold_count(oracle_mod):
    """Every (scale, bf16 magnitude <= block max) pair, both signs: the code
    is the count of thresholds t*s passed by |x| (exact products in fp64),
    with ties resolved toward the even code."""
    best = _largest_amax_per_scale()
    assert sorted(best) == list(range(1, 127))
    mags = all_bf16_magnitudes()
    rows, scales = [], []
    for sc, amax_bits in best.items():
        v = mags[mags <= amax_bits]
        for sign in (0, 0x8000):
            blk = np.empty((v.size, 2), np.uint16)
            blk[:, 0] = amax_bits
            blk[:, 1] = v | sign
            rows.append(blk)
            scales.append(np.full(v.size, sc))
    blocks = np.concatenate(rows)
    want_sc = np.concatenate(scales)
    codes, sc, xhat = oracle_mod.quantize(blocks)
    assert np.array_equal(sc[:, 0].astype(np.int64), want_sc)
    s = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()[want_sc]
    x = np.abs(bf16_to_f64(blocks[:, 1]))
    count = np.zeros(x.size, np.int64)
    ties = 0
    for t, up in _THRESHOLDS:
        tau = t * s
        count += (x >= tau) if up else (x > tau)
        ties += int(np.sum(x == tau))
    want_code = count | np.where(blocks[:, 1] & 0x8000, 8, 0)
    assert np.array_equal(codes[:, 1].astype(np.int64), want_code)
    assert ties > 500                      # exact E2M1 ties are exercised
    assert blocks.shape[0] > 3_000_000
    # dequantised value = signed E2M1 magnitude times the scale
    mag = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])[count]
    assert np.array_equal(np.abs(xhat[:, 1]), mag * s)


def test_element_rule_exact_rational_sample(oracle_mod):
    """A seeded sample of the same pairs against the exact checker."""
    rng = np.random.default_rng(7)
    best = _largest_amax_per_scale()
    mags = all_bf16_magnitudes()
    blocks = []
    for sc, amax_bits in best.items():
        v = mags[mags <= amax_bits]
        pick = rng.choice(v, size=min(40, v.size), replace=False)
        for p in pick:
            blocks.append([amax_bits, int(p) | (0x8000 if rng.random() < 0.5 else 0)])
    blocks = np.array(blocks, np.uint16)
    codes, sc, xhat = oracle_mod.quantize(blocks)
    for i, blk in enumerate(blocks):
        c, s, d = ex.encode_block([int(b) for b in blk])
        assert sc[i, 0] == s
        assert codes[i].tolist() == c
        assert [Fraction(float(z)) for z in xhat[i]] == d


# ---------------------------------------------------------- tiny brute force

def _small_values():
    """bf16 values with at most 3 significant bits in [2^-12, 2^12], both
    signs, and zero."""
    out = [0x0000, 0x8000]
    for e in range(-12, 13):
        for m in (0x00, 0x20, 0x40, 0x60):           # 1.00, 1.01, 1.10, 1.11
            bits = ((e + 127) << 7) | m
            out += [bits, bits | 0x8000]
    return out


def test_brute_force_tiny_blocks(oracle_mod):
    vals = _small_values()
    rng = np.random.default_rng(11)
    sub = [vals[i] for i in rng.choice(len(vals), 24, replace=False)] + [0x3F80, 0xBFC0]
    cases = [[v] for v in vals]
    cases += [list(p) for p in itertools.product(vals[::3], repeat=2)]
    cases += [list(p) for p in itertools.product(sub, repeat=3)]
    for blk in cases:
        codes, sc, xhat = oracle_mod.quantize_block(np.array(blk, np.uint16))
        c, s, d = ex.encode_block(blk)
        assert (codes.tolist(), sc) == (c, s), blk
        assert [Fraction(float(z)) for z in xhat] == d, blk


# --------------------------------------------------- hand-derived vectors

def _bits(values):
    return torch.tensor(values, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# Each vector: a block (rest of the 16 channels zero), the scale code, the
# codes of the listed channels, the packed bytes of those channels, and the
# dequantised values.  Derivations, by hand from the E2M1/E4M3 tables:
VECTORS = [
    # exact grid: amax 6 -> 6/6 = 1 = E4M3 0x38; every element is an E2M1 value
    # times 1, so it round-trips unchanged
    ("exact grid", [6, -4, 3, -2, 1.5, 1, 0.5, 0, -6, 4, -3, 2, -1.5, -1, -0.5, 0], 0x38,
     [0x7, 0xE, 0x5, 0xC, 0x3, 0x2, 0x1, 0x0, 0xF, 0x6, 0xD, 0x4, 0xB, 0xA, 0x9, 0x0],
     [0xE7, 0xC5, 0x23, 0x01, 0x6F, 0x4D, 0xAB, 0x09],
     [6, -4, 3, -2, 1.5, 1, 0.5, 0, -6, 4, -3, 2, -1.5, -1, -0.5, 0]),
    # 1/6 = 0.1667 lies between 0.15625 and 0.171875 (2^-3 x 1.25, x 1.375),
    # nearer the latter: code (4<<3)|3 = 0x23; 1/0.171875 = 5.82 > 5 -> 6
    ("amax one", [1], 0x23, [0x7], [0x07], [1.03125]),
    # 20/6 = 3.33 -> 3.25 (0x45); 20/3.25 = 6.15 saturates to 6; 1/3.25 = 0.31
    # > 0.25 -> 0.5; 0.5/3.25 and smaller round to 0 (negative keeps its sign)
    ("outlier sets the block scale", [20, 1, -1, 0.5, -0.5, 0.25, 0.30078125], 0x45,
     [0x7, 0x1, 0x9, 0x0, 0x8, 0x0, 0x0], [0x17, 0x09, 0x08],
     [19.5, 1.625, -1.625, 0, 0, 0, 0]),
    # 6.375/6 = 1.0625, exactly halfway between 1 (0x38) and 1.125 (0x39): even
    # code 0x38; 6.375/1 > 6 saturates to 6
    ("e4m3 tie, e2m1 saturation", [6.375], 0x38, [0x7], [0x07], [6]),
    # 3.75/6 = 0.625 = 0x32 exactly; quotients 6, 2.5, -5, 1.5: the ties 2.5 and
    # 5 go to the even codes 2 (0x4) and 4 (0x6)
    ("e2m1 ties, scale not a power of two", [3.75, 1.5625, -3.125, 0.9375], 0x32,
     [0x7, 0x4, 0xE, 0x3], [0x47, 0x3E], [3.75, 1.25, -2.5, 0.9375]),
    # all zero: amax/6 = 0 rounds to 0, replaced by the smallest subnormal 0x01
    ("all zero", [0] * 16, 0x01, [0] * 16, [0] * 8, [0] * 16),
    # 0.005/6 = 0.00083 < 2^-10 (half the smallest subnormal) -> 0 -> 0x01
    # (2^-9); 0.0050048828125 * 512 = 2.5625 -> 3; 0.00144 * 512 = 0.738 -> 0.5
    ("underflow to the smallest subnormal", [0.0050048828125, -0.00144195556640625], 0x01,
     [0x5, 0x9], [0x95], [0.005859375, -0.0009765625]),
    # 3000/6 = 500 saturates to 448 (0x7E); 3000/448 = 6.7 -> 6; -1/448 -> -0
    ("saturate both", [3000, -1], 0x7E, [0x7, 0x8], [0x87], [2688, 0]),
    # 1.40625/6 = 0.234375 = 0x27 exactly; quotients 6, 2.5, -1.25, 5: ties go
    # to 2, -1 and 4 (a reciprocal-multiply would push them up)
    ("ties broken by a reciprocal", [1.40625, 0.5859375, -0.29296875, 1.171875], 0x27,
     [0x7, 0x4, 0xA, 0x6], [0x47, 0x6A], [1.40625, 0.46875, -0.234375, 0.9375]),
]


@pytest.mark.parametrize("name,vals,scale,codes,packed,deq", VECTORS, ids=[v[0] for v in VECTORS])
def test_hand_derived_vectors(oracle_mod, name, vals, scale, codes, packed, deq):
    x = np.zeros(16, np.uint16)
    x[:len(vals)] = _bits(vals)
    nib, sc, xhat = oracle_mod.quantize(x.reshape(1, 16))
    assert sc[0, 0] == scale
    n = len(codes)
    assert nib[0, :n].tolist() == codes
    assert oracle_mod.pack_nibbles(nib[0])[: len(packed)].tolist() == packed
    assert xhat[0, :len(deq)].tolist() == [float(d) for d in deq]


# ----------------------------------------------------------------- invariants

def _random_blocks(n, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, 16, generator=g) * scale
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_exact_round_trip_of_representable_values(oracle_mod):
    """A block of E2M1 values times an E4M3 scale, with one element at +-6s,
    encodes to exactly those codes and decodes to itself."""
    rng = np.random.default_rng(3)
    e2 = oracle_mod.e2m1_table()
    for sc in range(8, 127):                     # normal scales: 6s keeps the scale code
        s = oracle_mod.e4m3_value(sc)
        codes = rng.integers(0, 16, 16)
        codes[rng.integers(0, 16)] = 7 | (8 if rng.random() < .5 else 0)
        vals = np.where(codes & 8, -1, 1) * e2[codes & 7] * s
        bits = _bits(vals.tolist())
        nib, scd, xhat = oracle_mod.quantize(bits.reshape(1, 16))
        assert scd[0, 0] == sc
        # zero magnitudes keep the sign of the bf16 zero they came from
        assert np.array_equal(nib[0] & 7, codes & 7)
        assert np.array_equal(xhat[0], vals)


def test_sign_symmetry(oracle_mod):
    x = _random_blocks(4096, 5, 3.0)
    n1, s1, d1 = oracle_mod.quantize(x)
    n2, s2, d2 = oracle_mod.quantize(x ^ np.uint16(0x8000))
    assert np.array_equal(s1, s2)
    assert np.array_equal(n1 ^ 8, n2)
    assert np.array_equal(d1, -d2)


def test_power_of_two_scaling(oracle_mod):
    """Multiplying a block by 2^k (normal, unsaturated scale range) keeps the
    codes and moves the scale code's exponent by k."""
    x = _random_blocks(2048, 9)
    n1, s1, d1 = oracle_mod.quantize(x)
    ok = (s1[:, 0] >= 0x18) & (s1[:, 0] <= 0x60)
    for k in (-2, 1, 3):
        xf = bf16_to_f64(x) * 2.0 ** k
        xk = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        n2, s2, d2 = oracle_mod.quantize(xk)
        assert np.array_equal(n1[ok], n2[ok])
        assert np.array_equal(s1[ok].astype(int) + 8 * k, s2[ok].astype(int))
        assert np.array_equal(d1[ok] * 2.0 ** k, d2[ok])


def test_idempotent_for_normal_scales(oracle_mod):
    x = _random_blocks(8192, 13, 2.0)
    n1, s1, d1 = oracle_mod.quantize(x)
    y = torch.from_numpy(d1).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    n2, s2, d2 = oracle_mod.quantize(y)
    normal = s1[:, 0] >= 8
    assert normal.all()
    assert np.array_equal(s1, s2)
    assert np.array_equal(n1, n2)
    assert np.array_equal(d1, d2)


def test_dequantize_matches_encoder_output(oracle_mod):
    x = _random_blocks(1024, 17, 5.0).reshape(64, 256)
    nib, sc, xhat = oracle_mod.quantize(x)
    assert np.array_equal(oracle_mod.dequantize(nib, sc), xhat)


def test_short_last_block(oracle_mod):
    """A row whose length is not a multiple of 16 ends in a shorter block,
    quantised on its own (as slicing a row in 16s does)."""
    x = _random_blocks(8, 21).reshape(-1)[:40].reshape(2, 20)
    nib, sc, _ = oracle_mod.quantize(x)
    assert sc.shape == (2, 2)
    for r in range(2):
        c, s, _ = ex.encode_block([int(b) for b in x[r, 16:]])
        assert sc[r, 1] == s and nib[r, 16:].tolist() == c


def test_rejects_non_finite(oracle_mod):
    x = np.zeros((1, 16), np.uint16)
    x[0, 3] = 0x7F80                               # +inf
    with pytest.raises(ValueError):
        oracle_mod.quantize(x)


def test_outlier_channel_inflates_its_group(oracle_mod):
    """One large channel sets its group's scale and flushes most of the
    group's other channels to zero, while the neighbouring group keeps a
    fine scale ("Week 6 -- FP4 KV Caches and Bounded Replay", Core Concepts)."""
    import fp4kv_workloads as wl
    w = wl.WORKLOADS["tiny_d64_ctx256"]
    k = wl.kv_tokens(w, 1, 0, "k", 0, w.context)
    nib, sc, _ = oracle_mod.quantize(wl.bf16_bits(k))
    s = oracle_mod.e4m3_table()[sc[:, 0, :]]
    ratio = np.median(s[:, 0] / s[:, 1])
    assert ratio > 4                      # ~20 x |N(0,1)| against the max of 16 |N(0,1)|
    x = np.abs(k.float().numpy()[:, 0, :16])
    assert np.mean(np.argmax(x, axis=1) == 7) > 0.9
    zero_frac = np.mean((nib[:, 0, :16] & 7)[:, [c for c in range(16) if c != 7]] == 0)
    zero_frac_next = np.mean((nib[:, 0, 16:32] & 7) == 0)
    assert zero_frac > 0.35 and zero_frac > 4 * zero_frac_next
