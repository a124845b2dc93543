"""fp4kv_decode_attention_noalloc: decode attention whose partial results go
to the library's static workspace instead of a caller's.  Its output must
equal fp4kv_decode_attention's bit for bit (the same kernels on the same
inputs), on consecutive calls that reuse the static workspace with a smaller
input the second time, and a plan larger than the static workspace is refused
on the host before any HIP call."""
import ctypes

import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_workloads as wl


def _say(msg):
    print(msg, flush=True)


def _case(lens, Hkv, G, D, seed):
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    maxp = max(1, max(-(-n // 64) for n in lens))
    table = torch.randperm(B * maxp, generator=g).to(torch.int32).reshape(B, maxp)
    L = fk.cache_layout(Hkv, D, B * maxp)
    cache = torch.zeros((L.cache_bytes,), dtype=torch.uint8, device="cuda")
    for b, n in enumerate(lens):
        if n > 0:
            k = (torch.randn(n, Hkv, D, generator=g) * 2).to(torch.bfloat16)
            v = torch.randn(n, Hkv, D, generator=g).to(torch.bfloat16)
            fk.quantize_append(L, k.cuda(), v.cuda(), wl.slots_for(table, b, 0, n).cuda(), cache)
    q = torch.randn(B, Hkv * G, D, generator=g).to(torch.bfloat16).cuda()
    return L, cache, table.cuda(), torch.tensor(lens, dtype=torch.int32).cuda(), q


@pytest.mark.gpu
def test_noalloc_equals_workspace_call_on_consecutive_calls():
    """Two calls in a row (the second smaller, with fewer partials) and a
    single-partial call after them: each equals decode_attention with a
    workspace of its own."""
    cases = [([3000, 0, 1, 65, 4096, 1000, 64, 2500], 2, 8, 128, 16, 31),
             ([700, 129, 2], 1, 4, 128, 0, 32),
             ([4096, 3000], 2, 16, 128, 8, 33),
             ([900, 0, 300], 1, 4, 64, 4, 34)]
    for lens, Hkv, G, D, splits, seed in cases:
        L, cache, pt, sl, q = _case(lens, Hkv, G, D, seed)
        plan = fk.decode_plan(L, len(lens), Hkv * G, pt.shape[1], splits)
        _say(f"noalloc: lens {lens} Hkv {Hkv} G {G} D {D} splits {splits} -> partials {plan.partials}")
        out = torch.full((len(lens), Hkv * G, D), float("nan"), dtype=torch.float32, device="cuda")
        fk.decode_attention_noalloc(L, cache, q, sl, pt, num_splits=splits, out=out)
        ws = torch.full((plan.workspace_bytes,), 0xC3, dtype=torch.uint8, device="cuda")
        ref = fk.decode_attention(L, cache, q, sl, pt, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (lens, splits)


@pytest.mark.gpu
def test_noalloc_on_a_second_stream():
    L, cache, pt, sl, q = _case([2000, 333, 1], 2, 8, 128, 41)
    ref = fk.decode_attention(L, cache, q, sl, pt, num_splits=12)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = fk.decode_attention_noalloc(L, cache, q, sl, pt, num_splits=12)
    s.synchronize()
    assert torch.equal(out, ref)


def test_noalloc_refuses_a_plan_larger_than_the_static_workspace():
    """Host-side: nothing is launched (aligned stand-in device addresses)."""
    L = fk.cache_layout(8, 128, 64)
    lib = fk.library()
    ok = 0x10000
    big_batch, hq, maxp, splits = 1024, 64, 512, 64
    need = fk.decode_plan(L, big_batch, hq, maxp, splits).workspace_bytes
    assert need > fk.NOALLOC_WORKSPACE_BYTES
    assert lib.fp4kv_decode_attention_noalloc(ctypes.byref(L), ok, ok, big_batch, hq, ok, ok, maxp,
                                              ctypes.c_float(0.1), splits, ok, None) == fk.ERR_WORKSPACE_TOO_SMALL
    # the other host checks of decode_attention apply as well
    assert lib.fp4kv_decode_attention_noalloc(ctypes.byref(L), ok, ok, 2, 32, ok, ok, 8, ctypes.c_float(0.1),
                                              0, None, None) == fk.ERR_INVALID_ARGUMENT
    assert lib.fp4kv_decode_attention_noalloc(ctypes.byref(L), ok, ok, 2, 32, ok, ok, 8, ctypes.c_float(0.1),
                                              0, ok + 4, None) == fk.ERR_MISALIGNED
    assert lib.fp4kv_decode_attention_noalloc(ctypes.byref(L), ok, ok, 0, 32, ok, ok, 8, ctypes.c_float(0.1),
                                              0, ok, None) == fk.OK
    # the 32-sequence, 32K-context batch at 64 chunks fits
    assert fk.decode_plan(fk.cache_layout(8, 128, 32 * 512), 32, 64, 512, 64).workspace_bytes <= \
        fk.NOALLOC_WORKSPACE_BYTES
