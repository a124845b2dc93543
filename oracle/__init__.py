"""CPU oracle for the FP4 (E2M1 elements, E4M3 scale per 16 channels) KV cache,
for its FP8 E4M3 variant with one scale per tensor, and for the formats of
the bit-width sweep (integers and FP8 E4M3 with an fp16 scale per token or per
channel, the unquantised bf16 cache).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg use it; the product library never imports, loads or calls it,
and it shares no code with the HIP path.  The arithmetic lives in
``fp4kv_oracle.c`` (plain C, exact rounding, fp64 attention); this module only
marshals numpy arrays into it, plus the page's cost model, which is plain
arithmetic.

Sources (page title, section):
  * "Quantising the KV cache" (numerics-explained), Code section: the block
    quantiser excerpt -- blocks of 16 channels, scale = E4M3(amax / 6) rounded
    to nearest even with saturation, zero scale replaced by the smallest E4M3
    subnormal, elements = E2M1(x / s) * s.
  * Same page, Maths section: cost per number = b + s/g bits (4 + 8/16 = 4.5
    for this format); a token holds 2 x layers x KV heads x head dim numbers.
  * Same page, Code and Concept sections: quantised K and V replace the real
    ones ahead of an unchanged attention; Q stays unquantised.
  * Same page, Concept section, results table: FP8 E4M3 with one scale per
    tensor, 8 bits per number.

Parity status: every function here is pinned by the CPU tests (format tables,
exhaustive scale and element rules against independent exact checkers and a
library FP8 conversion, brute force on tiny blocks, printed cost figures,
attention special cases and a library attention routine).  The pages' logit
drift and top-1 figures are "parity unpinned": they need a model that is not
available.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def lib():
    """The compiled oracle; built with gcc on first use if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        L = ctypes.CDLL(_build.LIBRARY)
        L.fp4kv_oracle_e2m1_value.restype = ctypes.c_double
        L.fp4kv_oracle_e2m1_value.argtypes = [ctypes.c_int]
        L.fp4kv_oracle_e4m3_value.restype = ctypes.c_double
        L.fp4kv_oracle_e4m3_value.argtypes = [ctypes.c_int]
        L.fp4kv_oracle_quantize_block.restype = ctypes.c_int
        L.fp4kv_oracle_quantize_block.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p]
        L.fp4kv_oracle_quantize_rows.restype = ctypes.c_int
        L.fp4kv_oracle_quantize_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int]
        L.fp4kv_oracle_attention.restype = ctypes.c_int
        L.fp4kv_oracle_attention.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        L.fp4kv_oracle_quantize_fp8.restype = ctypes.c_int
        L.fp4kv_oracle_quantize_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                                ctypes.c_void_p]
        L.fp4kv_oracle_attention_fp8.restype = ctypes.c_int
        L.fp4kv_oracle_attention_fp8.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                 ctypes.c_int64, ctypes.c_double, ctypes.c_double,
                                                 ctypes.c_double, ctypes.c_void_p]
        L.fp4kv_oracle_attention_fp8_batch.restype = ctypes.c_int
        L.fp4kv_oracle_attention_fp8_batch.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                       ctypes.c_void_p, ctypes.c_void_p,
                                                       ctypes.c_void_p, ctypes.c_void_p,
                                                       ctypes.c_int64, ctypes.c_double,
                                                       ctypes.c_double, ctypes.c_double,
                                                       ctypes.c_void_p, ctypes.c_int]
        L.fp4kv_oracle_attention_batch.restype = ctypes.c_int
        L.fp4kv_oracle_attention_batch.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_void_p, ctypes.c_void_p,
                                                   ctypes.c_int64, ctypes.c_int64,
                                                   ctypes.c_double, ctypes.c_void_p, ctypes.c_int]
        L.fp4kv_oracle_fp16_value.restype = ctypes.c_double
        L.fp4kv_oracle_fp16_value.argtypes = [ctypes.c_int]
        L.fp4kv_oracle_quantize_int.restype = ctypes.c_int
        L.fp4kv_oracle_quantize_int.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                ctypes.c_void_p, ctypes.c_void_p]
        L.fp4kv_oracle_quantize_fp8_groups.restype = ctypes.c_int
        L.fp4kv_oracle_quantize_fp8_groups.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                                       ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                                       ctypes.c_void_p]
        L.fp4kv_oracle_attention_values.restype = ctypes.c_int
        L.fp4kv_oracle_attention_values.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                                    ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                                    ctypes.c_int64, ctypes.c_double, ctypes.c_void_p]
        L.fp4kv_oracle_attention_values_batch.restype = ctypes.c_int
        L.fp4kv_oracle_attention_values_batch.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                                          ctypes.c_void_p, ctypes.c_void_p,
                                                          ctypes.c_void_p, ctypes.c_void_p,
                                                          ctypes.c_int64, ctypes.c_double,
                                                          ctypes.c_void_p, ctypes.c_int]
        _LIB = L
    return _LIB


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def as_bf16_bits(x) -> np.ndarray:
    """bf16 data as a uint16 numpy array of bit patterns (torch bf16 tensors
    or uint16/int16 arrays)."""
    if hasattr(x, "dtype") and str(getattr(x, "dtype")) == "torch.bfloat16":
        import torch
        return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    a = np.asarray(x)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected bf16 bit patterns (uint16)")
    return np.ascontiguousarray(a)


# ------------------------------------------------------------------ formats

def e2m1_value(code: int) -> float:
    """Magnitude of a 3-bit E2M1 code."""
    return lib().fp4kv_oracle_e2m1_value(int(code))


def e4m3_value(code: int) -> float:
    """Magnitude of a 7-bit E4M3 (OCP FN) code, 0..126."""
    return lib().fp4kv_oracle_e4m3_value(int(code))


def e2m1_table() -> np.ndarray:
    return np.array([e2m1_value(c) for c in range(8)], dtype=np.float64)


def e4m3_table() -> np.ndarray:
    return np.array([e4m3_value(c) for c in range(127)], dtype=np.float64)


# ---------------------------------------------------------------- quantiser

def quantize_block(x_bits):
    """One block of 1..16 bf16 values -> (codes[n], scale_code, xhat[n])."""
    x = as_bf16_bits(x_bits).ravel()
    n = x.size
    if not 1 <= n <= 16:
        raise ValueError("a block holds 1..16 values")
    nib = np.zeros(n, np.uint8)
    sc = np.zeros(1, np.uint8)
    xhat = np.zeros(n, np.float64)
    rc = lib().fp4kv_oracle_quantize_block(_ptr(x), n, _ptr(nib), _ptr(sc), _ptr(xhat))
    if rc:
        raise ValueError("non-finite input")
    return nib, int(sc[0]), xhat


def quantize(x_bits, want_xhat=True, n_threads=None):
    """Quantise the last axis of a bf16 array in blocks of 16 channels.

    Returns (codes uint8 [..., L] one nibble per byte with the sign in bit 3,
    scale codes uint8 [..., ceil(L/16)], xhat float64 [..., L] or None)."""
    x = as_bf16_bits(x_bits)
    shape = x.shape
    L = shape[-1]
    rows = int(np.prod(shape[:-1], dtype=np.int64)) if len(shape) > 1 else 1
    nb = (L + 15) // 16
    nib = np.empty(shape, np.uint8)
    sc = np.empty(shape[:-1] + (nb,), np.uint8)
    xhat = np.empty(shape, np.float64) if want_xhat else None
    rc = lib().fp4kv_oracle_quantize_rows(_ptr(x), rows, L, _ptr(nib), _ptr(sc),
                                          _ptr(xhat) if want_xhat else None,
                                          n_threads or default_threads())
    if rc:
        raise ValueError("non-finite input" if rc == -1 else "bad arguments")
    return nib, sc, xhat


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two codes per byte along the last axis: the even channel in the low
    nibble, the odd channel in the high nibble (the packing this library
    stores; the pages push dequantised numbers and never pack)."""
    c = np.asarray(codes, np.uint8)
    return (c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E2M1(code) * E4M3(scale), signed by bit 3 of the code, in float64."""
    e2 = e2m1_table()
    e4 = np.concatenate([e4m3_table(), [np.nan]])
    c = np.asarray(codes, np.uint8)
    s = np.repeat(np.asarray(scales, np.uint8), 16, axis=-1)[..., : c.shape[-1]]
    mag = e2[c & 7] * e4[s & 0x7F]
    return np.where(c & 8, -mag, mag)


def quantize_fp8(x_bits, scale):
    """FP8 E4M3 with one scale per tensor ("Quantising the KV cache", Concept,
    results table): codes uint8 of the same shape, sign in bit 7, magnitude
    RNE_sat_E4M3(|x| / scale) for a finite positive fp32 scale."""
    x = as_bf16_bits(x_bits)
    codes = np.empty(x.shape, np.uint8)
    s = np.float32(scale)
    rc = lib().fp4kv_oracle_quantize_fp8(_ptr(x), x.size, ctypes.c_float(s), _ptr(codes))
    if rc:
        raise ValueError("non-finite input or scale")
    return codes


def dequantize_fp8(codes, scale) -> np.ndarray:
    """+-E4M3(code) * scale in float64 (scale taken as fp32)."""
    e4 = np.concatenate([e4m3_table(), [np.nan]])
    c = np.asarray(codes, np.uint8)
    mag = e4[c & 0x7F] * float(np.float32(scale))
    return np.where(c & 0x80, -mag, mag)


# ---------------------------------------------------------------- attention

def attention(q_bits, k_codes, k_scales, v_codes, v_scales, scale):
    """fp64 attention of G bf16 query rows [G][D] over T tokens whose K and V
    are given as codes [T][D] and scale codes [T][D/16]; returns [G][D]."""
    q = as_bf16_bits(q_bits)
    G, D = q.shape
    kc = np.ascontiguousarray(k_codes, np.uint8)
    ks = np.ascontiguousarray(k_scales, np.uint8)
    vc = np.ascontiguousarray(v_codes, np.uint8)
    vs = np.ascontiguousarray(v_scales, np.uint8)
    T = kc.shape[0]
    out = np.zeros((G, D), np.float64)
    rc = lib().fp4kv_oracle_attention(_ptr(q), G, D, T, _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                                      D, D // 16, float(scale), _ptr(out))
    if rc:
        raise ValueError("bad arguments")
    return out


def decode_attention(q_bits, k_codes, k_scales, v_codes, v_scales, seq_lens, scale,
                     heads=None, n_threads=None):
    """Decode attention over a batch, from the oracle's own codes.

    q_bits:   [B][Hq][D] bf16 bit patterns.
    k_codes:  per sequence b, uint8 [>= len_b][Hkv][D] (one code per byte);
    k_scales: per sequence b, uint8 [>= len_b][Hkv][D/16]; v_* likewise.
    seq_lens: [B] context lengths.
    heads:    optional list of (b, kv_head) pairs to compute (others stay 0).
    Query head h reads KV head h // (Hq / Hkv) (reading: consecutive query
    heads share a KV head).  Returns float64 [B][Hq][D]."""
    q = as_bf16_bits(q_bits)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_codes[0]).shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), np.float64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hkv)]
    keep = []
    qp, Tp, knp, ksp, vnp, vsp, op = [], [], [], [], [], [], []
    for (b, h) in heads:
        kc = np.ascontiguousarray(k_codes[b], np.uint8)
        ks = np.ascontiguousarray(k_scales[b], np.uint8)
        vc = np.ascontiguousarray(v_codes[b], np.uint8)
        vs = np.ascontiguousarray(v_scales[b], np.uint8)
        qg = np.ascontiguousarray(q[b, h * G:(h + 1) * G])
        ob = np.zeros((G, D), np.float64)
        keep += [kc, ks, vc, vs, qg, ob]
        qp.append(_ptr(qg))
        Tp.append(int(seq_lens[b]))
        knp.append(_ptr(kc) + h * D)
        ksp.append(_ptr(ks) + h * (D // 16))
        vnp.append(_ptr(vc) + h * D)
        vsp.append(_ptr(vs) + h * (D // 16))
        op.append((b, h, ob))
    n = len(qp)
    P = ctypes.c_void_p * max(n, 1)
    T_arr = np.array(Tp if n else [0], np.int64)
    outs = P(*[_ptr(o[2]) for o in op]) if n else P()
    rc = lib().fp4kv_oracle_attention_batch(
        n, G, D, P(*qp), _ptr(T_arr), P(*knp), P(*ksp), P(*vnp), P(*vsp),
        Hkv * D, Hkv * (D // 16), float(scale), outs, n_threads or default_threads())
    if rc:
        raise ValueError("bad arguments")
    for (b, h, ob) in op:
        out[b, h * G:(h + 1) * G] = ob
    return out


def attention_fp8(q_bits, k_codes, v_codes, k_scale, v_scale, scale):
    """fp64 attention of G bf16 query rows [G][D] over T tokens of FP8 codes
    [T][D] with per-tensor scales; returns [G][D]."""
    q = as_bf16_bits(q_bits)
    G, D = q.shape
    kc = np.ascontiguousarray(k_codes, np.uint8)
    vc = np.ascontiguousarray(v_codes, np.uint8)
    out = np.zeros((G, D), np.float64)
    rc = lib().fp4kv_oracle_attention_fp8(_ptr(q), G, D, kc.shape[0], _ptr(kc), _ptr(vc), D,
                                          float(np.float32(k_scale)), float(np.float32(v_scale)),
                                          float(scale), _ptr(out))
    if rc:
        raise ValueError("bad arguments")
    return out


def decode_attention_fp8(q_bits, k_codes, v_codes, k_scale, v_scale, seq_lens, scale,
                         heads=None, n_threads=None):
    """decode_attention for an FP8 cache: k_codes / v_codes per sequence b,
    uint8 [>= len_b][Hkv][D]; per-tensor scales k_scale, v_scale."""
    q = as_bf16_bits(q_bits)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_codes[0]).shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), np.float64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hkv)]
    keep, qp, Tp, kp, vp, op = [], [], [], [], [], []
    for (b, h) in heads:
        kc = np.ascontiguousarray(k_codes[b], np.uint8)
        vc = np.ascontiguousarray(v_codes[b], np.uint8)
        qg = np.ascontiguousarray(q[b, h * G:(h + 1) * G])
        ob = np.zeros((G, D), np.float64)
        keep += [kc, vc, qg, ob]
        qp.append(_ptr(qg))
        Tp.append(int(seq_lens[b]))
        kp.append(_ptr(kc) + h * D)
        vp.append(_ptr(vc) + h * D)
        op.append((b, h, ob))
    n = len(qp)
    P = ctypes.c_void_p * max(n, 1)
    T_arr = np.array(Tp if n else [0], np.int64)
    outs = P(*[_ptr(o[2]) for o in op]) if n else P()
    rc = lib().fp4kv_oracle_attention_fp8_batch(
        n, G, D, P(*qp), _ptr(T_arr), P(*kp), P(*vp), Hkv * D, float(np.float32(k_scale)),
        float(np.float32(v_scale)), float(scale), outs, n_threads or default_threads())
    if rc:
        raise ValueError("bad arguments")
    for (b, h, ob) in op:
        out[b, h * G:(h + 1) * G] = ob
    return out


# ------------------------------------------- integer formats (bit-width sweep)

def fp16_value(code: int) -> float:
    return lib().fp4kv_oracle_fp16_value(int(code))


def fp16_table() -> np.ndarray:
    """Magnitudes of the finite fp16 codes 0 .. 0x7BFF."""
    return np.array([fp16_value(c) for c in range(0x7C00)], np.float64)


GRANULARITIES = ("token", "channel")


def quantize_int(x_bits, bits: int, granularity: str):
    """Symmetric bits-bit integer codes with one fp16 scale per group
    ("Quantising the KV cache", Concept section, results table: INT8 / INT4 /
    INT2 per token and per channel).

    x_bits: bf16 [T][H][D] of one sequence.  granularity "token": a group is
    one token's D channels of one head, scales [T][H]; "channel": a group is
    one channel of one head across the T tokens, scales [H][D].
    Returns (codes int8 [T][H][D], scale codes uint16 (fp16 bit patterns))."""
    x = as_bf16_bits(x_bits)
    if x.ndim != 3:
        raise ValueError("expected [T][H][D]")
    T, H, D = x.shape
    codes = np.zeros(x.shape, np.int8)
    if granularity == "token":
        scales = np.zeros((T, H), np.uint16)
        args = (T * H, D, D, 1)
    elif granularity == "channel":
        scales = np.zeros((H, D), np.uint16)
        args = (H * D, T, 1, H * D)
    else:
        raise ValueError("granularity is 'token' or 'channel'")
    if T == 0:
        return codes, scales
    rc = lib().fp4kv_oracle_quantize_int(_ptr(x), *args, int(bits), _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("bad arguments or non-finite input")
    return codes, scales


def dequantize_int(codes, scales, granularity: str) -> np.ndarray:
    """code * fp16(scale) in float64 (exact: at most 7 + 11 significant bits)."""
    c = np.asarray(codes, np.int8).astype(np.float64)
    s = np.asarray(scales, np.uint16).view(np.float16).astype(np.float64)
    if granularity == "token":
        return c * s[..., None]
    if granularity == "channel":
        return c * s[None]
    raise ValueError("granularity is 'token' or 'channel'")


def _group_args(shape, granularity):
    T, H, D = shape
    if granularity == "token":
        return np.zeros((T, H), np.uint16), (T * H, D, D, 1)
    if granularity == "channel":
        return np.zeros((H, D), np.uint16), (H * D, T, 1, H * D)
    raise ValueError("granularity is 'token' or 'channel'")


def quantize_fp8_groups(x_bits, granularity: str):
    """FP8 E4M3 codes with one fp16 scale per group: the finer FP8 scale
    granularities ("KV Cache Quantisation", Common questions; groups as in
    "Quantising the KV cache", Concept section).  Scale = fp16 nearest-even
    of amax / 448 (zero -> the smallest fp16 subnormal), code = sign bit |
    E4M3 nearest-even, saturating, of |x| / s.

    x_bits: bf16 [T][H][D] of one sequence; groups as in quantize_int.
    Returns (codes uint8 [T][H][D], scale codes uint16 (fp16 bit patterns))."""
    x = as_bf16_bits(x_bits)
    if x.ndim != 3:
        raise ValueError("expected [T][H][D]")
    codes = np.zeros(x.shape, np.uint8)
    scales, args = _group_args(x.shape, granularity)
    if x.shape[0] == 0:
        return codes, scales
    rc = lib().fp4kv_oracle_quantize_fp8_groups(_ptr(x), *args, _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("bad arguments or non-finite input")
    return codes, scales


def dequantize_fp8_groups(codes, scales, granularity: str) -> np.ndarray:
    """+-E4M3(code) * fp16(scale) in float64 (exact: 4 + 11 significant bits)."""
    c = np.asarray(codes, np.uint8)
    mag = e4m3_table()[np.minimum(c & 0x7F, 126)]
    val = np.where(c & 0x80, -mag, mag)
    s = np.asarray(scales, np.uint16).view(np.float16).astype(np.float64)
    if granularity == "token":
        return val * s[..., None]
    if granularity == "channel":
        return val * s[None]
    raise ValueError("granularity is 'token' or 'channel'")


def bf16_values(x_bits) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (the unquantised cache)."""
    x = as_bf16_bits(x_bits)
    return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_values(q_bits, k, v, scale):
    """fp64 attention of G bf16 query rows [G][D] over T tokens of exact K and
    V values (float64 [T][D]); returns [G][D]."""
    q = as_bf16_bits(q_bits)
    G, D = q.shape
    k = np.ascontiguousarray(k, np.float64)
    v = np.ascontiguousarray(v, np.float64)
    out = np.zeros((G, D), np.float64)
    rc = lib().fp4kv_oracle_attention_values(_ptr(q), G, D, k.shape[0], _ptr(k), _ptr(v), D,
                                             float(scale), _ptr(out))
    if rc:
        raise ValueError("bad arguments")
    return out


def decode_attention_values(q_bits, k_vals, v_vals, seq_lens, scale, heads=None, n_threads=None):
    """decode_attention over exact K and V values: k_vals / v_vals per
    sequence b, float64 [>= len_b][Hkv][D].  Query head h reads KV head
    h // (Hq / Hkv).  Returns float64 [B][Hq][D]."""
    q = as_bf16_bits(q_bits)
    B, Hq, D = q.shape
    Hkv = np.asarray(k_vals[0]).shape[1]
    if Hq % Hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), np.float64)
    if heads is None:
        heads = [(b, h) for b in range(B) for h in range(Hkv)]
    keep, qp, Tp, kp, vp, op = [], [], [], [], [], []
    for (b, h) in heads:
        kb = np.ascontiguousarray(k_vals[b], np.float64)
        vb = np.ascontiguousarray(v_vals[b], np.float64)
        qg = np.ascontiguousarray(q[b, h * G:(h + 1) * G])
        ob = np.zeros((G, D), np.float64)
        keep += [kb, vb, qg, ob]
        qp.append(_ptr(qg))
        Tp.append(int(seq_lens[b]))
        kp.append(_ptr(kb) + h * D * 8)
        vp.append(_ptr(vb) + h * D * 8)
        op.append((b, h, ob))
    n = len(qp)
    P = ctypes.c_void_p * max(n, 1)
    T_arr = np.array(Tp if n else [0], np.int64)
    outs = P(*[_ptr(o[2]) for o in op]) if n else P()
    rc = lib().fp4kv_oracle_attention_values_batch(
        n, G, D, P(*qp), _ptr(T_arr), P(*kp), P(*vp), Hkv * D, float(scale), outs,
        n_threads or default_threads())
    if rc:
        raise ValueError("bad arguments")
    for (b, h, ob) in op:
        out[b, h * G:(h + 1) * G] = ob
    return out


# --------------------------------------------------------------- cost model

def bits_per_number(elem_bits: float, scale_bits: float, group: float) -> float:
    """Bits per cached number with one scale of scale_bits per group values
    ("Quantising the KV cache", Maths section): b + s/g."""
    return elem_bits + (scale_bits / group if group else 0.0)


def numbers_per_token(n_layers: int, n_kv_heads: int, head_dim: int) -> int:
    """K and V numbers a token adds to the cache (same section):
    2 x layers x KV heads x head dim."""
    return 2 * n_layers * n_kv_heads * head_dim


def fp8_cache_bytes(n_tokens: int, n_layers: int, n_kv_heads: int, head_dim: int) -> float:
    """Resident bytes of an FP8 E4M3 cache with one scale per tensor: 8 bits
    per number (the per-tensor scale is negligible per number)."""
    return n_tokens * numbers_per_token(n_layers, n_kv_heads, head_dim) * bits_per_number(8, 0, 0) / 8


def fp4_cache_bytes(n_tokens: int, n_layers: int, n_kv_heads: int, head_dim: int) -> float:
    """Resident bytes of an FP4 cache (E2M1 + an E4M3 scale per 16): 4.5 bits
    per number over every token's K and V numbers."""
    return n_tokens * numbers_per_token(n_layers, n_kv_heads, head_dim) * bits_per_number(4, 8, 16) / 8
