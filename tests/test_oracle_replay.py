"""Pins for the oracle of the exact-versus-bounded replay study (CPU only).

"Week 6 -- FP4 KV Caches and Bounded Replay", Core Concepts and Lecture
notes: replaying about L * n_win tokens rebuilds the sliding-window states
exactly; replaying only the last n_win tokens is approximate.  The pins are
the receptive-field facts (exact replay equals the full run bit for bit in
float64; with one layer bounded replay is exact too; with several it is
not), a closed form for a window of one token, and the bf16 rounding
against torch's conversion."""
import numpy as np
import pytest
import torch

import fp4kv_workloads as wl
from oracle import toy_swa as ts


def test_bf16_round_matches_library():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(100000, generator=g) * torch.exp(torch.randn(100000, generator=g) * 8)
    ref = x.to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ts.bf16_round(x.double().numpy()), ref)
    # ties: exactly halfway values go to the even neighbour
    base = np.array([1.0, 1.0078125, 3.0, -5.5], np.float64)          # bf16 values
    half_ulp = np.array([2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -6])
    got = ts.bf16_round(base + half_ulp)
    want = torch.tensor(base + half_ulp, dtype=torch.float32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", ["toy_swa_l4_w32", "toy_swa_l2_w16"])
@pytest.mark.parametrize("fmt", ["fp8", "fp4", "bf16"])
def test_exact_replay_is_exact_and_bounded_is_not(name, fmt):
    net = wl.TOY_NETS[name]
    w, x = wl.toy_weights(net, 1), wl.toy_inputs(net, 1)
    ref, exact, bounded = ts.replay_study(net, w, x, fmt)
    assert np.array_equal(exact, ref)
    err = ts.relative_errors(bounded, ref)
    assert err.min() > 1e-6
    # one token fewer than the receptive field is no longer exact
    N = x.shape[1]
    r, _ = ts.replay_lengths(net)
    short = ts.run(net, w, x, N - r + 1, N, fmt)[:, -1]
    assert not np.array_equal(short, ref)


def test_one_layer_bounded_replay_is_exact():
    net = wl.TOY_NETS["toy_swa_l1_w32"]
    w, x = wl.toy_weights(net, 1), wl.toy_inputs(net, 1)
    for fmt in ("fp8", "fp4"):
        ref, exact, bounded = ts.replay_study(net, w, x, fmt)
        assert np.array_equal(bounded, ref) and np.array_equal(exact, ref)


def test_window_of_one_token_closed_form():
    """With window 1 each head attends to its own token only: one layer maps
    h to h + (v of the head's KV head, per query head) W_o."""
    net = wl.ToyNet("w1", layers=1, q_heads=4, kv_heads=2, head_dim=128, window=1, batch=2, tokens=3)
    w, x = wl.toy_weights(wl.TOY_NETS["toy_swa_l4_w32"], 3)[:1], wl.toy_inputs(net, 3)
    wq, wk, wv, wo = (np.asarray(m, np.float64) for m in w[0])
    out = ts.run(net, w, x, 0, 3, "bf16")
    h = np.asarray(x, np.float64)
    u = h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True))
    v = ts.bf16_round(u @ wv).reshape(2, 3, 2, 128)
    attn = v[:, :, [0, 0, 1, 1]].reshape(2, 3, 512)                 # query head j reads KV head j // 2
    np.testing.assert_allclose(out, h + attn @ wo, rtol=1e-12, atol=1e-12)


def test_error_grows_with_depth():
    """More layers behind the first: bounded replay misses more context."""
    errs = []
    for L in (2, 4):
        net = wl.ToyNet("depth", layers=L, q_heads=2, kv_heads=2, head_dim=128, window=8, batch=4, tokens=48)
        w, x = wl.toy_weights(net, 5), wl.toy_inputs(net, 5)
        ref, exact, bounded = ts.replay_study(net, w, x, "bf16")
        assert np.array_equal(exact, ref)
        errs.append(float(ts.relative_errors(bounded, ref).mean()))
    assert errs[0] < errs[1]


@pytest.mark.parametrize("fmt", ["fp8", "fp4", "bf16"])
def test_run_with_given_rows_reproduces_run(fmt):
    """Fed the rows run() projects, run_with_rows() reproduces its hidden
    states bit for bit (the two share the attention arithmetic, not the
    projections); rows that are not bf16 are refused."""
    net = wl.ToyNet("rows", layers=2, q_heads=4, kv_heads=2, head_dim=128, window=6, batch=2, tokens=20)
    w, x = wl.toy_weights(net, 4), wl.toy_inputs(net, 4)
    rows = []
    ref = ts.run(net, w, x, 3, 20, fmt, record=rows)
    assert len(rows) == 17 and len(rows[0]) == 2
    out, attns = ts.run_with_rows(net, w, x, 3, 20, rows, fmt)
    assert np.array_equal(out, ref)
    assert attns.shape == (17, 2, 2, 4, 128) and np.isfinite(attns).all()
    bad = [[(q + 1e-9, k, v) for q, k, v in layer] for layer in rows]
    with pytest.raises(AssertionError):
        ts.run_with_rows(net, w, x, 3, 20, bad, fmt)
