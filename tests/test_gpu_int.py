"""GPU parity of the integer formats of the bit-width sweep: codes and fp16
scales bit-exact against the oracle's, decode attention within 1e-3 per row
of the oracle's fp64 attention over the same stored values (and, for bits
16, over the unquantised bf16 values)."""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_harness as hx
import fp4kv_workloads as wl
import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _say(msg):
    print(msg, flush=True)


def _check_quantize(x, bits, gran):
    """x bf16 [B][T][H][D] on the CPU; compare the GPU's codes and scales
    with the oracle's, sequence by sequence."""
    B, T, H, D = x.shape
    codes, scales = fk.int_quantize(x.cuda(), bits, gran)
    torch.cuda.synchronize()
    got = hx.unpack_int_codes(codes, bits, D)
    gs = hx.int_scales_host(scales, gran)
    for b in range(B):
        c, s = oracle.quantize_int(wl.bf16_bits(x[b]), bits, gran)
        assert np.array_equal(got[b], c), (bits, gran, b)
        assert np.array_equal(gs[b], s), (bits, gran, b)


def _all_bf16_rows(D, sign_flip):
    allb = np.array([b for b in range(0x10000) if (b >> 7) & 0xFF != 0xFF], np.uint16)
    if sign_flip:
        allb = allb[::-1].copy()
    n = -(-allb.size // D) * D
    pad = np.zeros(n, np.uint16)
    pad[: allb.size] = allb
    return torch.from_numpy(pad.view(np.int16).reshape(1, -1, 1, D)).view(torch.bfloat16)


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("D", [64, 128])
def test_every_bf16_value_per_token(bits, D):
    """Every finite bf16 pattern, in order and reversed, D to a row: every
    scale range (subnormal fallback, normal, saturated) and every element."""
    for flip in (False, True):
        x = _all_bf16_rows(D, flip)
        _say(f"int quantize per token: every bf16, bits {bits}, D {D}, reversed {flip}")
        _check_quantize(x, bits, "token")


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_exact_ties_and_fp16_midpoints(bits):
    """Rows whose elements sit exactly on integer + 1/2 of the scale, and
    amax values whose amax / qmax is exactly an fp16 rounding midpoint (the
    case the quantiser settles with an FMA)."""
    qmax = (1 << (bits - 1)) - 1
    rows = []
    for e in (-20, -3, 0, 5):
        s = 2.0 ** e
        for k in range(qmax):
            rows.append([qmax * s, (k + 0.5) * s, -(k + 0.5) * s] + [0.0] * 61)
    # amax / qmax exactly an fp16 rounding midpoint.  From a bf16 amax that
    # happens only among the fp16 subnormals ((k + 1/2) * 2^-24): a normal
    # midpoint has 12 significant bits, more than amax / qmax can carry.
    for k in range(0, 40):
        rows.append([qmax * (k + 0.5) * 2.0 ** -24, 2.0 ** -26] + [0.0] * 62)
    x = torch.tensor(rows, dtype=torch.float32)
    xb = x.to(torch.bfloat16)
    keep = (xb.float() == x).all(dim=1)                  # rows that are exact in bf16
    xb = xb[keep].reshape(1, -1, 1, 64)
    _say(f"int quantize: {xb.shape[1]} tie and midpoint rows, bits {bits}")
    _check_quantize(xb, bits, "token")


@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("shape", [(2, 300, 3, 128), (1, 1, 1, 64), (3, 77, 2, 64), (1, 4096, 8, 128)])
def test_per_channel_and_per_token_random(bits, shape):
    """Seeded rows with per-channel magnitudes over four decades (so both
    granularities see very different groups), a ragged token count, and a
    sequence of a single token."""
    B, T, H, D = shape
    g = torch.Generator().manual_seed(B * 1000 + T + bits)
    f = torch.exp(torch.empty(H, D).uniform_(-5, 5, generator=g))
    x = (torch.randn(B, T, H, D, generator=g) * f).to(torch.bfloat16)
    for gran in ("token", "channel"):
        _say(f"int quantize: {shape}, bits {bits}, per {gran}")
        _check_quantize(x, bits, gran)


def test_bf16_copy_and_zero_tokens():
    x = torch.randn(2, 37, 3, 64).to(torch.bfloat16)
    codes, scales = fk.int_quantize(x.cuda(), 16, "token")
    torch.cuda.synchronize()
    assert scales.numel() == 0
    back = codes.view(torch.int16).view(torch.bfloat16).cpu().permute(0, 2, 1, 3)
    assert torch.equal(back.view(torch.int16), x.view(torch.int16))
    empty = torch.empty(2, 0, 3, 64, dtype=torch.bfloat16, device="cuda")
    c0, s0 = fk.int_quantize(empty, 4, "channel")
    assert c0.numel() == 0


def _oracle_values(x, bits, gran):
    """float64 [T][H][D] of one sequence as stored (or exact bf16 for 16)."""
    bits_ = wl.bf16_bits(x)
    if bits == 16:
        return oracle.bf16_values(bits_)
    if bits == fk.INT_FP8_E4M3:
        c, s = oracle.quantize_fp8_groups(bits_, gran)
        return oracle.dequantize_fp8_groups(c, s, gran)
    c, s = oracle.quantize_int(bits_, bits, gran)
    return oracle.dequantize_int(c, s, gran)


def _decode_case(B, T, H, G, D, bits, kg, vg, splits, seed):
    g = torch.Generator().manual_seed(seed)
    f = torch.exp(torch.empty(H, D).uniform_(-1.5, 1.5, generator=g))
    k = (torch.randn(B, T, H, D, generator=g) * f * 2).to(torch.bfloat16)
    v = torch.randn(B, T, H, D, generator=g).to(torch.bfloat16)
    q = torch.randn(B, H * G, D, generator=g).to(torch.bfloat16)
    kq = fk.int_quantize(k.cuda(), bits, kg)
    vq = fk.int_quantize(v.cuda(), bits, vg)
    out = fk.int_decode_attention(q.cuda(), bits, kq, vq, T, kg, vg, num_splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    kv = [_oracle_values(k[b], bits, kg) for b in range(B)]
    vv = [_oracle_values(v[b], bits, vg) for b in range(B)]
    ref = oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, [T] * B, D ** -0.5)
    return out, ref


@pytest.mark.parametrize("bits,kg,vg", [(16, "token", "token"), (8, "token", "token"), (4, "token", "token"),
                                        (4, "channel", "token"), (2, "token", "token"),
                                        (2, "channel", "token"), (8, "token", "channel")])
@pytest.mark.parametrize("T,splits", [(1, 0), (255, 1), (257, 0), (1000, 3)])
def test_decode_matches_oracle(bits, kg, vg, T, splits):
    for (G, D) in ((4, 128), (16, 64)):
        _say(f"int decode: bits {bits}, K per {kg}, V per {vg}, T {T}, splits {splits}, G {G}, D {D}")
        out, ref = _decode_case(2, T, 2, G, D, bits, kg, vg, splits, seed=T + bits + G)
        err = float(hx.row_rel_error(out, ref).max())
        _say(f"  worst per-row relative error {err:.3e}")
        assert err <= TOL


def test_decode_empty_context_and_odd_groups():
    for G in (1, 3, 9):
        out, ref = _decode_case(2, 0, 1, G, 128, 8, "token", "token", 0, seed=G)
        assert not out.any()
        out, ref = _decode_case(1, 300, 3, G, 128, 4, "channel", "token", 2, seed=G)
        assert float(hx.row_rel_error(out, ref).max()) <= TOL


def test_decode_workload_shape():
    """The 8-sequence, 4096-token, 8-KV-head workload (four key channels per
    head x10), INT4 with K per channel: two sequences checked."""
    w = wl.WORKLOADS["gqa4_b8_ctx4k"]
    T = 4096
    k = torch.stack([wl.kv_tokens(w, 2, b, "k", 0, T) for b in range(w.batch)])
    v = torch.stack([wl.kv_tokens(w, 2, b, "v", 0, T) for b in range(w.batch)])
    q = wl.queries(w, 2)
    _say("int decode: gqa4_b8_ctx4k, INT4 K per channel, V per token")
    kq = fk.int_quantize(k.cuda(), 4, "channel")
    vq = fk.int_quantize(v.cuda(), 4, "token")
    out = fk.int_decode_attention(q.cuda(), 4, kq, vq, T, "channel", "token")
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    heads = [(b, h) for b in (0, 5) for h in range(w.kv_heads)]
    kv = [_oracle_values(k[b], 4, "channel") if b in (0, 5) else np.zeros((1, w.kv_heads, 128))
          for b in range(w.batch)]
    vv = [_oracle_values(v[b], 4, "token") if b in (0, 5) else np.zeros((1, w.kv_heads, 128))
          for b in range(w.batch)]
    ref = oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, [T] * w.batch, 128 ** -0.5, heads=heads)
    err = max(float(hx.row_rel_error(out[b], ref[b]).max()) for b in (0, 5))
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("bits,kg", [(16, "token"), (8, "token"), (4, "channel"), (2, "token"),
                                     (fk.INT_FP8_E4M3, "token")])
def test_decode_rising_scores_long_split(bits, kg):
    """Scores that grow along the sequence, so each wave's running maximum
    moves block after block, over one split per (sequence, head) of 5,000
    tokens (every wave takes many blocks, the last one partial)."""
    B, T, H, G, D = 2, 5000, 2, 8, 128
    g = torch.Generator().manual_seed(bits)
    q = torch.randn(B, H * G, D, generator=g)
    direction = q.view(B, H, G, D).mean(2)                      # [B][H][D]
    ramp = torch.linspace(0, 6, T).view(1, T, 1, 1)
    k = (torch.randn(B, T, H, D, generator=g) + ramp * direction.view(B, 1, H, D)).to(torch.bfloat16)
    v = torch.randn(B, T, H, D, generator=g).to(torch.bfloat16)
    q = q.to(torch.bfloat16)
    _say(f"int decode, rising scores: bits {bits}, K per {kg}, T {T}, one split")
    kq = fk.int_quantize(k.cuda(), bits, kg)
    vq = fk.int_quantize(v.cuda(), bits, "token")
    out = fk.int_decode_attention(q.cuda(), bits, kq, vq, T, kg, "token", num_splits=1)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    kv = [_oracle_values(k[b], bits, kg) for b in range(B)]
    vv = [_oracle_values(v[b], bits, "token") for b in range(B)]
    ref = oracle.decode_attention_values(wl.bf16_bits(q), kv, vv, [T] * B, D ** -0.5)
    err = float(hx.row_rel_error(out, ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("bits,kg,vg", [(16, "token", "token")] +
                         [(b, g, g) for b in (8, 4, 2, fk.INT_FP8_E4M3) for g in ("token", "channel")])
def test_decode_single_token_returns_stored_values_exactly(bits, kg, vg):
    """With one token of context every head's softmax weight is exactly 1,
    so each output row must be the stored V row itself, bit for bit: this
    pins the value path's channel order, the code conversion and the removal
    of the INT4 / INT2 offset (all exact by construction)."""
    for G, D in ((4, 128), (16, 64)):
        B, H = 3, 2
        g = torch.Generator().manual_seed(bits + G)
        k = torch.randn(B, 1, H, D, generator=g).to(torch.bfloat16)
        v = (torch.randn(B, 1, H, D, generator=g) * torch.exp(torch.empty(H, D).uniform_(-2, 2, generator=g))
             ).to(torch.bfloat16)
        q = torch.randn(B, H * G, D, generator=g).to(torch.bfloat16)
        _say(f"int decode, one token: bits {bits}, K per {kg}, V per {vg}, G {G}, D {D}")
        kq = fk.int_quantize(k.cuda(), bits, kg)
        vq = fk.int_quantize(v.cuda(), bits, vg)
        out = fk.int_decode_attention(q.cuda(), bits, kq, vq, 1, kg, vg)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        for b in range(B):
            vv = _oracle_values(v[b], bits, vg)[0]                    # [H][D], float64, exact in fp32
            want = np.repeat(vv, G, axis=0).astype(np.float32)
            assert np.array_equal(out[b], want), (b, np.abs(out[b] - want).max())
