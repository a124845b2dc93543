"""GPU parity of the FP8 E4M3 formats with an fp16 scale per token or per
channel (the finer FP8 scale granularities of the bit-width sweep): codes and
scales bit-exact against the oracle's, decode attention within 1e-3 per row
of the oracle's fp64 attention over the same stored values."""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_harness as hx
import fp4kv_workloads as wl
import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-3
FP8 = fk.INT_FP8_E4M3


def _say(msg):
    print(msg, flush=True)


def _check_quantize(x, gran):
    """x bf16 [B][T][H][D] on the CPU; the GPU's codes and scales against the
    oracle's, sequence by sequence."""
    B, T, H, D = x.shape
    codes, scales = fk.int_quantize(x.cuda(), FP8, gran)
    torch.cuda.synchronize()
    got = np.ascontiguousarray(codes.cpu().numpy().transpose(0, 2, 1, 3))      # [B][T][H][D]
    gs = hx.int_scales_host(scales, gran)
    for b in range(B):
        c, s = oracle.quantize_fp8_groups(wl.bf16_bits(x[b]), gran)
        assert np.array_equal(got[b], c), (gran, b)
        assert np.array_equal(gs[b], s), (gran, b)


def _all_bf16_rows(D, reverse):
    allb = np.array([b for b in range(0x10000) if (b >> 7) & 0xFF != 0xFF], np.uint16)
    if reverse:
        allb = allb[::-1].copy()
    n = -(-allb.size // D) * D
    pad = np.zeros(n, np.uint16)
    pad[: allb.size] = allb
    return torch.from_numpy(pad.view(np.int16).reshape(1, -1, 1, D)).view(torch.bfloat16)


@pytest.mark.parametrize("D", [64, 128])
def test_every_bf16_value_per_token(D):
    """Every finite bf16 pattern, in order and reversed, D to a row: every
    scale range (subnormal fallback, normal, saturated) and every element."""
    for rev in (False, True):
        _say(f"fp8 per-group quantize: every bf16, D {D}, reversed {rev}")
        _check_quantize(_all_bf16_rows(D, rev), "token")


def test_exact_ties_and_fp16_midpoints():
    """Elements exactly halfway between two E4M3 magnitudes times the scale,
    and amax values whose amax / 448 is exactly an fp16 rounding midpoint
    (the cases the quantiser settles with an FMA)."""
    e4 = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    rows = []
    for s in (2.0 ** -20, 0.75, 1.0, 2.0 ** 5):
        for k in range(0, 126, 2):
            m0, m1 = (e4[k] + e4[k + 1]) / 2 * s, (e4[k + 1] + e4[k + 2]) / 2 * s if k + 2 < 127 else 0.0
            rows.append([448.0 * s, m0, -m0, m1, -m1] + [0.0] * 59)
    # from a bf16 amax, amax / 448 is an fp16 midpoint only among the fp16
    # subnormals ((k + 1/2) * 2^-24)
    for k in range(0, 40):
        rows.append([448.0 * (k + 0.5) * 2.0 ** -24, 2.0 ** -30, -(2.0 ** -31)] + [0.0] * 61)
    x = torch.tensor(rows, dtype=torch.float64)
    xb = x.to(torch.bfloat16)
    keep = (xb.double() == x).all(dim=1)                 # rows that are exact in bf16
    xb = xb[keep].reshape(1, -1, 1, 64)
    assert xb.shape[1] > 200
    _say(f"fp8 per-group quantize: {xb.shape[1]} tie and midpoint rows")
    _check_quantize(xb, "token")


@pytest.mark.parametrize("shape", [(2, 300, 3, 128), (1, 1, 1, 64), (3, 77, 2, 64), (1, 4096, 8, 128)])
def test_per_channel_and_per_token_random(shape):
    """Seeded rows with per-channel magnitudes over four decades, ragged
    token counts, and a sequence of a single token."""
    B, T, H, D = shape
    g = torch.Generator().manual_seed(B * 1000 + T)
    f = torch.exp(torch.empty(H, D).uniform_(-5, 5, generator=g))
    x = (torch.randn(B, T, H, D, generator=g) * f).to(torch.bfloat16)
    for gran in ("token", "channel"):
        _say(f"fp8 per-group quantize: {shape}, per {gran}")
        _check_quantize(x, gran)


def _values(x, gran):
    c, s = oracle.quantize_fp8_groups(wl.bf16_bits(x), gran)
    return oracle.dequantize_fp8_groups(c, s, gran)


def _decode_case(B, T, H, G, D, kg, vg, splits, seed):
    g = torch.Generator().manual_seed(seed)
    f = torch.exp(torch.empty(H, D).uniform_(-1.5, 1.5, generator=g))
    k = (torch.randn(B, T, H, D, generator=g) * f * 2).to(torch.bfloat16)
    v = torch.randn(B, T, H, D, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H * G, D, generator=g).to(torch.bfloat16)
    kq = fk.int_quantize(k.cuda(), FP8, kg)
    vq = fk.int_quantize(v.cuda(), FP8, vg)
    out = fk.int_decode_attention(q.cuda(), FP8, kq, vq, T, kg, vg, num_splits=splits)
    torch.cuda.synchronize()
    kv = [_values(k[b], kg) for b in range(B)]
    vv = [_values(v[b], vg) for b in range(B)]
    ref = oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, [T] * B, D ** -0.5)
    return out.cpu().numpy(), ref


@pytest.mark.parametrize("kg,vg", [("token", "token"), ("channel", "token"), ("token", "channel"),
                                   ("channel", "channel")])
@pytest.mark.parametrize("T,splits", [(1, 0), (255, 1), (257, 0), (1000, 3)])
def test_decode_matches_oracle(kg, vg, T, splits):
    for (G, D) in ((4, 128), (16, 64), (3, 128)):
        _say(f"fp8 per-group decode: K per {kg}, V per {vg}, T {T}, splits {splits}, G {G}, D {D}")
        out, ref = _decode_case(2, T, 2, G, D, kg, vg, splits, seed=T + G + D)
        err = float(hx.row_rel_error(out, ref).max())
        _say(f"  worst per-row relative error {err:.3e}")
        assert err <= TOL


def test_decode_empty_context():
    out, _ = _decode_case(2, 0, 1, 4, 128, "token", "token", 0, seed=1)
    assert not out.any()


def test_decode_workload_shape():
    """The 8-sequence, 4096-token, 8-KV-head workload (four key channels per
    head x10), FP8 with K per channel and V per token: two sequences checked."""
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    T = 4096
    k = torch.stack([wl.kv_tokens(w, 2, b, "k", 0, T) for b in range(w.batch)])
    v = torch.stack([wl.kv_tokens(w, 2, b, "v", 0, T) for b in range(w.batch)])
    q = wl.queries(w, 2)
    _say("fp8 per-group decode: gqa4_b8_ctx4k, K per channel, V per token")
    kq = fk.int_quantize(k.cuda(), FP8, "channel")
    vq = fk.int_quantize(v.cuda(), FP8, "token")
    out = fk.int_decode_attention(q.cuda(), FP8, kq, vq, T, "channel", "token")
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    heads = [(b, h) for b in (0, 5) for h in range(w.kv_heads)]
    kv = [_values(k[b], "channel") if b in (0, 5) else np.zeros((1, w.kv_heads, 128)) for b in range(w.batch)]
    vv = [_values(v[b], "token") if b in (0, 5) else np.zeros((1, w.kv_heads, 128)) for b in range(w.batch)]
    ref = oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, [T] * w.batch, 128 ** -0.5, heads=heads)
    err = max(float(hx.row_rel_error(out[b], ref[b]).max()) for b in (0, 5))
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL
