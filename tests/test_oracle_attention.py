"""Pins for the oracle's fp64 decode attention and the page's cost model (CPU only)."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import exact_checker as ex
import fp4kv_workloads as wl


def _bf16(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _rand_kv(oracle_mod, T, D, seed, scale=1.0, heads=None):
    g = torch.Generator().manual_seed(seed)
    shape = (T, D) if heads is None else (T, heads, D)
    k = _bf16(torch.randn(*shape, generator=g) * scale)
    v = _bf16(torch.randn(*shape, generator=g))
    kn, ks, kh = oracle_mod.quantize(k)
    vn, vs, vh = oracle_mod.quantize(v)
    return kn, ks, kh, vn, vs, vh


def _q(G, D, seed):
    g = torch.Generator().manual_seed(seed)
    return _bf16(torch.randn(G, D, generator=g))


def _qf(q):
    return (q.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_single_token_returns_its_value(oracle_mod):
    kn, ks, kh, vn, vs, vh = _rand_kv(oracle_mod, 1, 128, 1)
    out = oracle_mod.attention(_q(4, 128, 2), kn, ks, vn, vs, 128 ** -0.5)
    assert np.array_equal(out, np.repeat(vh, 4, 0))


def test_equal_keys_give_the_mean_value(oracle_mod):
    kn, ks, kh, vn, vs, vh = _rand_kv(oracle_mod, 37, 64, 3)
    kn[:] = kn[0]
    ks[:] = ks[0]
    out = oracle_mod.attention(_q(2, 64, 4), kn, ks, vn, vs, 0.125)
    np.testing.assert_allclose(out, np.repeat(vh.mean(0, keepdims=True), 2, 0), rtol=0, atol=1e-14)


def test_zero_query_gives_the_mean_value(oracle_mod):
    kn, ks, kh, vn, vs, vh = _rand_kv(oracle_mod, 53, 128, 5, scale=7.0)
    q = np.zeros((1, 128), np.uint16)
    out = oracle_mod.attention(q, kn, ks, vn, vs, 1.0)
    np.testing.assert_allclose(out[0], vh.mean(0), rtol=0, atol=1e-14)


def test_empty_context_gives_zeros(oracle_mod):
    kn, ks, kh, vn, vs, vh = _rand_kv(oracle_mod, 0, 64, 6)
    out = oracle_mod.attention(_q(3, 64, 7), kn, ks, vn, vs, 0.125)
    assert np.array_equal(out, np.zeros((3, 64)))


@pytest.mark.parametrize("T,D,kscale,scale", [(300, 64, 1.0, 0.125), (517, 128, 3.0, 128 ** -0.5),
                                            (64, 128, 20.0, 0.3)])
def test_matches_library_attention(oracle_mod, T, D, kscale, scale):
    """Same dequantised K and V (decoded by the Python dequantiser), attention
    by torch's scaled_dot_product_attention in float64."""
    kn, ks, kh, vn, vs, vh = _rand_kv(oracle_mod, T, D, 8 + T, scale=kscale)
    q = _q(4, D, 9)
    out = oracle_mod.attention(q, kn, ks, vn, vs, scale)
    K = torch.from_numpy(oracle_mod.dequantize(kn, ks))
    V = torch.from_numpy(oracle_mod.dequantize(vn, vs))
    ref = F.scaled_dot_product_attention(torch.from_numpy(_qf(q))[None], K[None], V[None], scale=scale)[0]
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_batch_gqa_mapping_matches_library_attention(oracle_mod):
    """Query head h attends to KV head h // G; checked against SDPA on K and V
    repeated per query head, over a batch with different lengths."""
    B, Hq, Hkv, D = 3, 8, 2, 64
    G = Hq // Hkv
    lens = [70, 1, 129]
    g = torch.Generator().manual_seed(10)
    q = _bf16(torch.randn(B, Hq, D, generator=g))
    kc, ksc, vc, vsc, kd, vd = [], [], [], [], [], []
    for b in range(B):
        k = _bf16(torch.randn(lens[b] + 5, Hkv, D, generator=g) * 2)   # 5 extra rows never read
        v = _bf16(torch.randn(lens[b] + 5, Hkv, D, generator=g))
        kn, ks, kh = oracle_mod.quantize(k)
        vn, vs, vh = oracle_mod.quantize(v)
        kc.append(kn); ksc.append(ks); vc.append(vn); vsc.append(vs); kd.append(kh); vd.append(vh)
    out = oracle_mod.decode_attention(q, kc, ksc, vc, vsc, lens, D ** -0.5)
    for b in range(B):
        K = torch.from_numpy(kd[b][:lens[b]]).permute(1, 0, 2).repeat_interleave(G, 0)
        V = torch.from_numpy(vd[b][:lens[b]]).permute(1, 0, 2).repeat_interleave(G, 0)
        Q = torch.from_numpy(_qf(q[b]))[:, None, :]
        ref = F.scaled_dot_product_attention(Q, K, V, scale=D ** -0.5)[:, 0]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_token_permutation_invariance(oracle_mod):
    kn, ks, kh, vn, vs, vh = _rand_kv(oracle_mod, 200, 128, 11)
    q = _q(8, 128, 12)
    out = oracle_mod.attention(q, kn, ks, vn, vs, 0.09)
    p = np.random.default_rng(0).permutation(200)
    out2 = oracle_mod.attention(q, kn[p], ks[p], vn[p], vs[p], 0.09)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-13)


def test_large_scores_stay_finite(oracle_mod):
    """Outlier keys push scores to hundreds; the max-subtracted softmax stays
    finite and concentrates on the top token."""
    kn, ks, kh, vn, vs, vh = _rand_kv(oracle_mod, 50, 64, 13, scale=200.0)
    q = _q(1, 64, 14)
    out = oracle_mod.attention(q, kn, ks, vn, vs, 1.0)
    z = _qf(q) @ kh.T
    assert np.isfinite(out).all()
    np.testing.assert_allclose(out[0], vh[np.argmax(z[0])], rtol=0, atol=1e-9)


# --------------------------------------------------------------- cost model

def test_cost_table_from_the_page(oracle_mod):
    """b + s/g reproduces every printed bits-per-number and % of FP16."""
    rows = ex.read_table("kv_cache_cost_table.txt")
    assert len(rows) == 8
    for fmt, bits, pct, b, s, g in rows:
        got = oracle_mod.bits_per_number(float(b), float(s), float(g))
        assert got == float(bits), fmt
        assert round(100.0 * got / 16, 1) == float(pct), fmt


def test_fp4_cost_figures(oracle_mod):
    bits = oracle_mod.bits_per_number(4, 8, 16)
    assert bits == 4.5
    assert bits / 16 == 0.28125                 # printed as 28.1% of FP16
    assert bits / 8 == 0.5625                   # a little over half of an FP8 cache
    # one token of one layer with 8 KV heads of 128: 2*8*128 numbers, 1152 bytes
    assert oracle_mod.numbers_per_token(1, 8, 128) == 2048
    assert oracle_mod.fp4_cache_bytes(1, 1, 8, 128) == 1152
    # the 32-sequence, 32768-token, 8-head, d=128 cache in the benchmark set
    w = wl.WORKLOADS["gqa8_b32_ctx32k"]
    assert oracle_mod.fp4_cache_bytes(w.batch * w.context, 1, w.kv_heads, w.head_dim) == 1_207_959_552
