"""Oracle of the exact-versus-bounded replay study in a toy sliding-window
network (TEST INFRASTRUCTURE ONLY: used by the tests and by the script that
writes tests/golden/replay_*.txt; the product path never imports it).

"Week 6 -- FP4 KV Caches and Bounded Replay" (Overview, Core Concepts,
Lecture notes, Lab): sliding-window (SWA) layers attend over the last n_win
tokens and keep that window's K and V (in FP8, as the page says local state
is kept); rebuilding the windows exactly means replaying about L * n_win
tokens through L layers, while bounded replay replays only the last n_win
tokens and accepts a small error.

The page gives no network, so the toy one is the plainest that has the
property (readings, stated again in the design notes):
  * L layers; layer l maps the hidden state h (width d = Hq * D) of token t
    to h + W_o . attn, attn = sliding-window attention of q = u W_q over the
    stored K, V of the last `window` tokens (t included) of that layer,
    u = h / rms(h) (an RMS normalisation without weights), k = u W_k,
    v = u W_v, Hq query heads over Hkv KV heads (query head j reads KV head
    j // (Hq / Hkv)), softmax scale 1/sqrt(D); no MLP, no positional code;
  * q, k and v are rounded to bf16 (the precision the cache and the decode
    kernels take), then k and v are stored in the cache format: FP8 E4M3 with
    one scale per tensor (6/448: a 6-sigma value of a unit-variance channel at
    the top of the range), FP4 E2M1 with an E4M3 scale per 16, or bf16
    (unquantised);
  * everything else in float64.
Receptive field: layer l's state at token t depends on tokens
t - l*(window-1) .. t, so replaying the last L*(window-1)+1 tokens from empty
windows rebuilds the final output exactly, and replaying the last `window`
tokens is exact for layer 1 only.
"""
import numpy as np

from . import dequantize_fp8, quantize, quantize_fp8

FP8_SCALE = np.float32(6.0 / 448.0)


def bf16_round(x) -> np.ndarray:
    """float64 -> nearest bf16 value (ties to even), as float64, by integer
    rounding of the float64 bit pattern (finite inputs)."""
    a = np.ascontiguousarray(x, np.float64)
    bits = a.view(np.uint64)
    # bf16 keeps 7 of float64's 52 fraction bits: drop 45, ties to even
    drop = np.uint64(45)
    half = np.uint64(1) << np.uint64(44)
    lsb = (bits >> drop) & np.uint64(1)
    rounded = ((bits + half - np.uint64(1) + lsb) >> drop) << drop
    out = rounded.view(np.float64)
    # values beyond the bf16 range or below its subnormals are not expected here
    return out


def _bf16_bits(x64) -> np.ndarray:
    """bf16 bit patterns of float64 values that are exactly bf16."""
    f32 = np.asarray(x64, np.float64).astype(np.float32)
    return (f32.view(np.uint32) >> 16).astype(np.uint16)


def _store(x64, fmt):
    """The values the cache holds for rows x64 [..., D] already in bf16."""
    if fmt == "bf16":
        return x64
    bits = _bf16_bits(x64)
    if fmt == "fp8":
        return dequantize_fp8(quantize_fp8(bits, FP8_SCALE), FP8_SCALE)
    if fmt == "fp4":
        return quantize(bits)[2]
    raise ValueError("format is bf16, fp8 or fp4")


def run(net, weights, x, start: int, end: int, fmt: str = "fp8", record=None) -> np.ndarray:
    """Final hidden states of tokens start .. end-1 ([B][end-start][d],
    float64), processing them one at a time from empty windows.  With a list
    `record`, appends for every token the (q, k, v) bf16 rows of each layer
    (the input run_with_rows takes)."""
    B = x.shape[0]
    Hq, Hkv, D, W = net.q_heads, net.kv_heads, net.head_dim, net.window
    G = Hq // Hkv
    ws = [tuple(np.asarray(m, np.float64) for m in layer) for layer in weights]
    xs = np.asarray(x, np.float64)
    kwin = [[[] for _ in range(B)] for _ in range(net.layers)]      # stored K rows [Hkv][D] per token
    vwin = [[[] for _ in range(B)] for _ in range(net.layers)]
    out = np.zeros((B, end - start, net.d_model))
    scale = D ** -0.5
    for t in range(start, end):
        h = xs[:, t].copy()
        for layer, (wq, wk, wv, wo) in enumerate(ws):
            u = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True))
            q = bf16_round(u @ wq).reshape(B, Hq, D)
            k_row = bf16_round(u @ wk).reshape(B, Hkv, D)
            v_row = bf16_round(u @ wv).reshape(B, Hkv, D)
            if record is not None:
                if layer == 0:
                    record.append([])
                record[-1].append((q, k_row, v_row))
            attn = _window_attention(q, _store(k_row, fmt), _store(v_row, fmt), kwin[layer], vwin[layer], W, G,
                                     scale)
            h = h + attn.reshape(B, Hq * D) @ wo
        out[:, t - start] = h
    return out


def _window_attention(q, k, v, kwin, vwin, W, G, scale):
    """One token's attention in one layer: appends the stored k, v rows
    [B][Hkv][D] to the per-sequence windows kwin, vwin and attends q
    [B][Hq][D] over their last W rows (query head j reads KV head j // G)."""
    B, Hq, D = q.shape
    attn = np.zeros((B, Hq, D))
    for b in range(B):
        kwin[b].append(k[b])
        vwin[b].append(v[b])
        kk = np.stack(kwin[b][-W:])                         # [n][Hkv][D]
        vv = np.stack(vwin[b][-W:])
        for j in range(Hq):
            z = scale * (kk[:, j // G] @ q[b, j])
            p = np.exp(z - z.max())
            attn[b, j] = (p @ vv[:, j // G]) / p.sum()
    return attn


def run_with_rows(net, weights, x, start: int, end: int, rows, fmt: str = "fp8"):
    """As run(), but with the bf16 q, k and v rows of every (token, layer)
    given instead of projected here: rows[t - start][layer] = (q [B][Hq][D],
    k [B][Hkv][D], v [B][Hkv][D]), values exactly bf16.  Compares another
    implementation's attention and residual stream with the oracle's on
    identical inputs to the cache, so that no rounding of a projection can
    flip a stored code.  Returns the final hidden states [B][end-start][d]
    and the attention outputs [end-start][L][B][Hq][D]."""
    B = x.shape[0]
    Hq, Hkv, D, W = net.q_heads, net.kv_heads, net.head_dim, net.window
    G = Hq // Hkv
    ws = [tuple(np.asarray(m, np.float64) for m in layer) for layer in weights]
    xs = np.asarray(x, np.float64)
    kwin = [[[] for _ in range(B)] for _ in range(net.layers)]
    vwin = [[[] for _ in range(B)] for _ in range(net.layers)]
    out = np.zeros((B, end - start, net.d_model))
    attns = np.zeros((end - start, net.layers, B, Hq, D))
    scale = D ** -0.5
    for t in range(start, end):
        h = xs[:, t].copy()
        for layer, (_, _, _, wo) in enumerate(ws):
            q, k, v = (np.asarray(r, np.float64) for r in rows[t - start][layer])
            assert np.array_equal(bf16_round(q), q) and np.array_equal(bf16_round(k), k), "rows must be bf16"
            attn = _window_attention(q, _store(k, fmt), _store(v, fmt), kwin[layer], vwin[layer], W, G, scale)
            attns[t - start, layer] = attn
            h = h + attn.reshape(B, Hq * D) @ wo
        out[:, t - start] = h
    return out, attns


def replay_lengths(net):
    """Tokens replayed to rebuild the last token's output: exactly
    (L*(window-1)+1) and bounded (window)."""
    return net.layers * (net.window - 1) + 1, net.window


def replay_study(net, weights, x, fmt: str = "fp8"):
    """Final output of the last token from the full run, from exact replay
    and from bounded replay; returns (ref, exact, bounded) [B][d]."""
    N = x.shape[1]
    r_exact, r_bounded = replay_lengths(net)
    ref = run(net, weights, x, 0, N, fmt)[:, -1]
    exact = run(net, weights, x, N - r_exact, N, fmt)[:, -1]
    bounded = run(net, weights, x, N - r_bounded, N, fmt)[:, -1]
    return ref, exact, bounded


def relative_errors(a, ref) -> np.ndarray:
    """Per sequence ||a - ref|| / ||ref|| (Euclidean norm over the hidden
    width)."""
    return np.linalg.norm(np.asarray(a) - ref, axis=-1) / np.linalg.norm(ref, axis=-1)
