"""The GPU bit-width sweep against the oracle's: each format's bits per
number equal, its mean and largest attention-output row error within 2e-3 of
the oracle's (each side's outputs are within 1e-3 per row of exact, so the
two error figures can differ by about twice that)."""
import pytest

import exact_checker as ex
import sweep

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,seed", [("tiny_d64_ctx256", 1), ("gqa4_b8_ctx4k", 2)])
def test_sweep_matches_oracle_table(name, seed):
    print(f"bit-width sweep on {name}, seed {seed}", flush=True)
    want = {r[0]: (float(r[1]), float(r[2]), float(r[3]))
            for r in ex.read_table(f"bitwidth_sweep_{name}.txt")}
    got = sweep.error_table(name, seed)
    assert [r[0] for r in got] == list(want)
    for fname, bpn, mean, mx in got:
        wb, wm, wx = want[fname]
        print(f"  {fname:36s} {bpn:8.4f} {mean:.4e} ({wm:.4e}) {mx:.4e} ({wx:.4e})", flush=True)
        assert bpn == pytest.approx(wb, abs=1e-6)
        assert abs(mean - wm) <= 2e-3 + 1e-3 * wm
        assert abs(mx - wx) <= 2e-3 + 1e-3 * wx
