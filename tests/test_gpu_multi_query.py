"""GPU parity of causal attention for several query tokens per sequence
(fp4kv_decode_multi_attention): query token i of S sees the first
len - (S - 1 - i) tokens; each query token's rows within 1e-3 of the
oracle's fp64 attention over that prefix, one query token identical to
decode_attention."""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_harness as hx
import fp4kv_workloads as wl
import kv_formats as kf
import oracle

pytestmark = pytest.mark.gpu
TOL = 1e-3


def _say(msg):
    print(msg, flush=True)


def _cache(lens, Hkv, D, fmt, seed):
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    maxp = max(1, max(-(-n // 64) for n in lens))
    table = torch.randperm(B * maxp, generator=g).to(torch.int32).reshape(B, maxp)
    L = kf.layout(fmt, Hkv, D, B * maxp)
    cache = torch.full((L.cache_bytes,), 0x7F, dtype=torch.uint8, device="cuda")
    kv = {}
    for b, n in enumerate(lens):
        k = (torch.randn(n, Hkv, D, generator=g) * 2).to(torch.bfloat16)
        v = torch.randn(n, Hkv, D, generator=g).to(torch.bfloat16)
        kv[b] = (k, v)
        if n:
            fk.quantize_append(L, k.cuda(), v.cuda(), wl.slots_for(table, b, 0, n).cuda(), cache)
    torch.cuda.synchronize()
    return L, cache, table, kv, g


def _reference(L, kv, lens, q, fmt, D, Hkv):
    """fp64 oracle attention of query token i over the first
    len - (S - 1 - i) tokens, from the oracle's own codes."""
    B, S, Hq, _ = q.shape
    ref = np.zeros((B, S, Hq, D))
    for i in range(S):
        li = [max(0, n - (S - 1 - i)) for n in lens]
        qi = wl.bf16_bits(q[:, i].contiguous())
        if fmt == "fp8t":
            kv_ = [kf.stored_values(fmt, L, kv[b][0]) if lens[b] else np.zeros((1, Hkv, D)) for b in range(B)]
            vv_ = [kf.stored_values(fmt, L, kv[b][1]) if lens[b] else np.zeros((1, Hkv, D)) for b in range(B)]
            ref[:, i] = oracle.decode_attention_values(qi, kv_, vv_, li, D ** -0.5)
        elif fmt == "fp8":
            ks, vs = L.params.k_scale, L.params.v_scale
            kc = [oracle.quantize_fp8(wl.bf16_bits(kv[b][0]), ks) if lens[b] else np.zeros((1, Hkv, D), np.uint8)
                  for b in range(B)]
            vc = [oracle.quantize_fp8(wl.bf16_bits(kv[b][1]), vs) if lens[b] else np.zeros((1, Hkv, D), np.uint8)
                  for b in range(B)]
            ref[:, i] = oracle.decode_attention_fp8(qi, kc, vc, ks, vs, li, D ** -0.5)
        else:
            kq = [oracle.quantize(wl.bf16_bits(kv[b][0]), want_xhat=False) if lens[b] else
                  (np.zeros((1, Hkv, D), np.uint8), np.ones((1, Hkv, D // 16), np.uint8), None) for b in range(B)]
            vq = [oracle.quantize(wl.bf16_bits(kv[b][1]), want_xhat=False) if lens[b] else
                  (np.zeros((1, Hkv, D), np.uint8), np.ones((1, Hkv, D // 16), np.uint8), None) for b in range(B)]
            ref[:, i] = oracle.decode_attention(qi, [x[0] for x in kq], [x[1] for x in kq],
                                                [x[0] for x in vq], [x[1] for x in vq], li, D ** -0.5)
    return ref


@pytest.mark.parametrize("fmt,D", [("fp4", 128), ("fp4", 64), ("fp8", 128), ("fp8", 64), ("fp8t", 128),
                                   ("fp8t", 64)])
@pytest.mark.parametrize("S,G", [(2, 8), (4, 4), (16, 1), (3, 5)])
@pytest.mark.parametrize("splits", [0, 1, 5])
def test_against_oracle(fmt, D, S, G, splits):
    lens = [0, 1, 3, 17, 64, 65, 130, 1000]
    Hkv = 2
    L, cache, table, kv, g = _cache(lens, Hkv, D, fmt, seed=S * 31 + G + D + splits)
    q = torch.randn(len(lens), S, Hkv * G, D, generator=g).to(torch.bfloat16)
    _say(f"multi-query: {fmt} D {D} S {S} G {G} splits {splits}")
    out = fk.decode_multi_attention(L, cache, q.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(),
                                    table.cuda(), num_splits=splits)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    ref = _reference(L, kv, lens, q, fmt, D, Hkv)
    # query tokens whose prefix is empty give zero rows
    for b, n in enumerate(lens):
        for i in range(S):
            if n - (S - 1 - i) <= 0:
                assert not out[b, i].any()
    err = float(hx.row_rel_error(out, ref).max())
    _say(f"  worst per-row relative error {err:.3e}")
    assert err <= TOL


@pytest.mark.parametrize("fmt,D", [("fp4", 128), ("fp4", 64), ("fp8", 128), ("fp8", 64), ("fp8t", 128),
                                   ("fp8t", 64)])
def test_one_query_token_is_decode_attention(fmt, D):
    lens = [5, 64, 700]
    L, cache, table, kv, g = _cache(lens, 2, D, fmt, seed=3)
    q = torch.randn(3, 1, 8, D, generator=g).to(torch.bfloat16)
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    a = fk.decode_multi_attention(L, cache, q.cuda(), lens_d, table.cuda())
    b = fk.decode_attention(L, cache, q[:, 0].contiguous().cuda(), lens_d, table.cuda())
    torch.cuda.synchronize()
    assert torch.equal(a[:, 0], b)


def test_too_many_columns_rejected():
    L = fk.cache_layout(2, 128, 4)
    cache = torch.zeros(L.cache_bytes, dtype=torch.uint8, device="cuda")
    q = torch.zeros(1, 3, 12, 128, dtype=torch.bfloat16, device="cuda")       # 3 tokens x group 6 = 18
    with pytest.raises(fk.Fp4KVError) as e:
        fk.decode_multi_attention(L, cache, q, torch.ones(1, dtype=torch.int32, device="cuda"),
                                  torch.zeros(1, 4, dtype=torch.int32, device="cuda"))
    assert e.value.status == fk.ERR_UNSUPPORTED
