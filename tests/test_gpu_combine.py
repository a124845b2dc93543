"""GPU numerics of fp4kv_decode_combine on hand-made partial results.

The merge of split partials is the definition in include/fp4kv.h: with
M = max_j m_j, out = sum_j o_j 2^(m_j - M) / sum_j l_j 2^(m_j - M), zero where
every partial is empty (m = -inf, l = 0; an empty partial's o is not
meaningful and must not reach the result, even when it holds NaN).  The library picks one of two
kernels by the partial count (one wave per row up to 32 partials, a
workgroup per row above), so the counts below straddle that boundary.  The
reference is the same formula in float64.
"""
import numpy as np
import pytest
import torch

import fp4_quantised_kv_amd as fk

pytestmark = pytest.mark.gpu


def _round_up(x, m):
    return (x + m - 1) // m * m


def _workspace(o, ml):
    """Pack o [B][P][H][D] and ml [B][P][H][2] (float32) into the workspace
    layout fp4kv_decode_split writes."""
    ob = o.astype(np.float32).tobytes()
    mb = ml.astype(np.float32).tobytes()
    off = _round_up(len(ob), 256)
    buf = np.zeros(off + _round_up(len(mb), 256), np.uint8)
    buf[: len(ob)] = np.frombuffer(ob, np.uint8)
    buf[off: off + len(mb)] = np.frombuffer(mb, np.uint8)
    return torch.from_numpy(buf).cuda()


def _reference(o, ml):
    m = ml[..., 0].astype(np.float64)                       # [B][P][H]
    l = ml[..., 1].astype(np.float64)
    M = m.max(axis=1, keepdims=True)                        # [B][1][H]
    with np.errstate(invalid="ignore"):
        w = np.where(np.isfinite(m), np.exp2(m - np.where(np.isfinite(M), M, 0.0)), 0.0)
    L = (l * w).sum(axis=1)                                 # [B][H]
    O = (o.astype(np.float64) * w[..., None]).sum(axis=1)   # [B][H][D]
    return np.where(L[..., None] > 0, O / np.where(L > 0, L, 1.0)[..., None], 0.0)


def _partials(rng, B, P, H, D, empty_frac, empty_o=0.0):
    m = rng.normal(0.0, 6.0, (B, P, H)).astype(np.float32)
    l = rng.uniform(0.5, 200.0, (B, P, H)).astype(np.float32)
    o = rng.normal(0.0, 30.0, (B, P, H, D)).astype(np.float32)
    empty = rng.random((B, P, H)) < empty_frac
    empty[0, :, 0] = True                                    # one row with no tokens at all
    m[empty] = -np.inf
    l[empty] = 0.0
    o[empty] = empty_o
    return o, np.stack([m, l], axis=-1)


@pytest.mark.parametrize("empty_o", [0.0, float("nan"), float("inf")])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("P", [1, 2, 5, 16, 17, 31, 32, 33, 70])
def test_combine_matches_definition(P, D, empty_o):
    """Empty partials' outputs hold zeros, NaN or infinity (what an
    unwritten workspace may hold): the result is the same."""
    rng = np.random.default_rng(1000 * P + D)
    B, H = 3, 5
    o, ml = _partials(rng, B, P, H, D, empty_frac=0.3, empty_o=empty_o)
    ws = _workspace(o, ml)
    out = fk.decode_combine(ws, B, H, D, P)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ref = _reference(np.where(np.isfinite(o), o, 0.0), ml)
    assert np.array_equal(got[0, 0], np.zeros(D))             # every partial empty -> zero row
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    err = np.abs(got - ref) / np.where(scale > 0, scale, 1.0)
    assert err.max() <= 1e-5, (P, D, float(err.max()))


@pytest.mark.parametrize("P", [16, 64])
def test_combine_many_rows(P):
    """Row counts that do not fill the last workgroup of the one-wave-per-row
    kernel (4 rows per workgroup), and a large batch."""
    rng = np.random.default_rng(7 + P)
    D = 128
    for B, H in ((1, 1), (1, 3), (7, 9), (64, 32)):
        o, ml = _partials(rng, B, P, H, D, empty_frac=0.1)
        out = fk.decode_combine(_workspace(o, ml), B, H, D, P)
        torch.cuda.synchronize()
        ref = _reference(o, ml)
        got = out.cpu().numpy().astype(np.float64)
        scale = np.abs(ref).max(axis=-1, keepdims=True)
        err = np.abs(got - ref) / np.where(scale > 0, scale, 1.0)
        assert err.max() <= 1e-5, (B, H, float(err.max()))
