"""Exact-rational re-derivation of the FP4 block encoding, for pinning the oracle.

This is a second, independent statement of the rounding rules, written a
different way from the oracle: values are Python Fractions, the nearest code
is found by scanning every code's exact distance (not by neighbouring
midpoints), bf16 bit patterns are decoded field by field, and the E4M3 value
table comes from torch's float8_e4m3fn dtype (a library decoder), while the
E2M1 table comes from the stored magnitudes in tests/golden.
"""
from fractions import Fraction
import os

import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append([c.strip() for c in line.split("|")])
    return rows


E2M1 = [Fraction(r[1]) for r in read_table("e2m1_magnitudes.txt")]
_e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
E4M3 = [Fraction(v) for v in _e4]


def bf16_fraction(bits: int) -> Fraction:
    """Exact value of a finite bf16 bit pattern, decoded field by field."""
    sign = -1 if bits & 0x8000 else 1
    exp = (bits >> 7) & 0xFF
    man = bits & 0x7F
    if exp == 0xFF:
        raise ValueError("not finite")
    if exp == 0:
        return sign * Fraction(man, 128) * Fraction(2) ** (-126)
    return sign * (1 + Fraction(man, 128)) * Fraction(2) ** (exp - 127)


def nearest_code(y: Fraction, table) -> int:
    """Nearest entry of an ascending table; exact ties go to the even code;
    anything at or above the last entry saturates to it."""
    if y >= table[-1]:
        return len(table) - 1
    best, best_d = None, None
    for code, v in enumerate(table):
        d = abs(y - v)
        if best is None or d < best_d or (d == best_d and code % 2 == 0):
            best, best_d = code, d
    return best


def nearest_code_sorted(y: Fraction, table) -> int:
    """Same result as nearest_code, by bisection (for long tables)."""
    if y >= table[-1]:
        return len(table) - 1
    lo, hi = 0, len(table) - 1          # table[lo] <= y < table[hi]
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if table[mid] <= y:
            lo = mid
        else:
            hi = mid
    dl, dh = y - table[lo], table[hi] - y
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if lo % 2 == 0 else hi


def scale_code(amax: Fraction) -> int:
    c = nearest_code_sorted(amax / 6, E4M3)
    return c if c != 0 else 1


def encode_block(bits_list):
    """bf16 bit patterns of one block -> (codes, scale code, dequantised)."""
    vals = [bf16_fraction(b) for b in bits_list]
    sc = scale_code(max(abs(v) for v in vals))
    s = E4M3[sc]
    codes, deq = [], []
    for b, v in zip(bits_list, vals):
        neg = 1 if b & 0x8000 else 0
        e = nearest_code(abs(v) / s, E2M1)
        codes.append(neg << 3 | e)
        deq.append((-1 if neg else 1) * E2M1[e] * s)
    return codes, sc, deq
