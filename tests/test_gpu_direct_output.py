"""GPU tests of the single-partial decode path.

When the plan gives one partial per row (contexts of at most four chunks),
the decode entry points let the split kernel write the final output rows
itself and launch no combine.  With one partial the combine's weight is
exactly 1, so the rows must equal those of the split + combine path
(fp4kv_decode_with_options with a separate combine kernel) for every kernel
and entry point."""

import pytest
import torch

import fp4_quantised_kv_amd as fk
import fp4kv_workloads as wl
import kv_formats as kf

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _cache(fmt, lens, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    B = len(lens)
    maxp = max(1, max(-(-(n + 1) // 64) for n in lens))
    table = torch.randperm(B * maxp, generator=g).to(torch.int32).reshape(B, maxp)
    L = kf.layout(fmt, Hkv, D, B * maxp)
    cache = torch.zeros((L.cache_bytes,), dtype=torch.uint8, device="cuda")
    for b, n in enumerate(lens):
        if n > 0:
            k = (torch.randn(n, Hkv, D, generator=g) * 2).to(torch.bfloat16)
            v = torch.randn(n, Hkv, D, generator=g).to(torch.bfloat16)
            fk.quantize_append(L, k.cuda(), v.cuda(), wl.slots_for(table, b, 0, n).cuda(), cache)
    torch.cuda.synchronize()
    return L, cache, table.cuda()


def _both(call, **kw):
    """(default finish, split + combine kernel) of the same call."""
    ref = fk.decode_with_options(*call, merge="combine_kernel", **kw)
    torch.cuda.synchronize()
    ref = ref.cpu()
    got = fk.decode_with_options(*call, **kw)
    torch.cuda.synchronize()
    return got.cpu(), ref


CASES = [
    # fmt, D, lens, Hkv, G, splits (<= 4 chunks: one partial), kernel
    ("fp4", 128, [256, 0, 1, 63, 64, 65, 200], 2, 8, 4, None),
    ("fp4", 128, [3000, 4096, 17], 2, 4, 4, None),
    ("fp4", 128, [1000, 2000], 1, 16, 3, None),
    ("fp4", 64, [256, 0, 65, 100], 1, 4, 4, None),
    ("fp4", 128, [1000, 3, 2000], 2, 8, 2, "valu"),
    ("fp4", 128, [1000, 3, 2000], 2, 8, 4, "mfma_direct"),
    ("fp8", 128, [1000, 0, 65, 3000], 2, 8, 4, None),
    ("fp8t", 128, [1000, 0, 65, 3000], 2, 8, 1, None),
    ("fp8", 64, [1000, 0, 65, 3000], 2, 4, 4, None),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_direct_output_equals_combine(case):
    fmt, D, lens, Hkv, G, splits, kernel = CASES[case]
    _say(f"single partial: {CASES[case]}")
    L, cache, pt = _cache(fmt, lens, Hkv, D, seed=400 + case)
    assert fk.decode_plan(L, len(lens), Hkv * G, pt.shape[1], splits).partials == 1
    g = torch.Generator().manual_seed(500 + case)
    q = torch.randn(len(lens), Hkv * G, D, generator=g).to(torch.bfloat16).cuda()
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    ws = torch.full((fk.decode_plan(L, len(lens), Hkv * G, pt.shape[1], splits).workspace_bytes,), 0xC3,
                    dtype=torch.uint8, device="cuda")
    got, ref = _both((L, cache, q, sl, pt), num_splits=splits, workspace=ws, kernel=kernel or "auto")
    assert torch.equal(got, ref)
    if kernel is None:
        plain = fk.decode_attention(L, cache, q, sl, pt, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(plain.cpu(), got)
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.equal(got[b], torch.zeros_like(got[b]))     # an empty sequence gives zero rows


def test_direct_output_multi_window_append():
    lens, Hkv, G, D = [3000, 65, 1500, 4096], 2, 4, 128
    L, cache, pt = _cache("fp4", lens, Hkv, D, seed=77)
    g = torch.Generator().manual_seed(78)
    q2 = torch.randn(len(lens), 2, Hkv * G, D, generator=g).to(torch.bfloat16).cuda()
    q1 = torch.randn(len(lens), Hkv * G, D, generator=g).to(torch.bfloat16).cuda()
    kn = torch.randn(len(lens), Hkv, D, generator=g).to(torch.bfloat16).cuda()
    vn = torch.randn(len(lens), Hkv, D, generator=g).to(torch.bfloat16).cuda()
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    for splits in (1, 4):
        got, ref = _both((L, cache, q2, sl, pt), num_splits=splits)
        assert torch.equal(got, ref), ("multi", splits)
        assert torch.equal(fk.decode_multi_attention(L, cache, q2, sl, pt, num_splits=splits).cpu(), got)
        got, ref = _both((L, cache, q2, sl, pt), window=700, num_splits=splits)
        assert torch.equal(got, ref), ("window", splits)
        assert torch.equal(fk.decode_window_attention(L, cache, q2, sl, pt, 700, num_splits=splits).cpu(), got)
        got, ref = _both((L, cache, q1, sl, pt), k_new=kn, v_new=vn, num_splits=splits)
        assert torch.equal(got, ref), ("append", splits)
        assert torch.equal(fk.decode_append_attention(L, cache, kn, vn, q1, sl, pt, num_splits=splits).cpu(), got)


def test_options_are_checked():
    """Kernels that do not serve the arguments are refused, before any launch."""
    lens, Hkv, G, D = [300, 65], 2, 4, 128
    L, cache, pt = _cache("fp4", lens, Hkv, D, seed=79)
    L8, cache8, pt8 = _cache("fp8", lens, Hkv, D, seed=79)
    q1 = torch.zeros(2, Hkv * G, D, dtype=torch.bfloat16, device="cuda")
    q2 = torch.zeros(2, 2, Hkv * G, D, dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32).cuda()
    for args, kw in [((L, cache, q2, sl, pt), dict(kernel="valu")),              # several query tokens
                     ((L, cache, q1, sl, pt), dict(kernel="valu", window=64)),    # a window
                     ((L8, cache8, q1, sl, pt8), dict(kernel="mfma_direct")),    # an FP8 cache
                     ((L8, cache8, q1, sl, pt8), dict(kernel="valu"))]:
        with pytest.raises(fk.Fp4KVError) as e:
            fk.decode_with_options(*args, **kw)
        assert e.value.status == fk.ERR_UNSUPPORTED
