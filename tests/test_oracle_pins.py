"""The oracle against its pins (see tests/oracle_pins.py for what each rests on)."""
import pytest

from oracle import moda_forward, moda_forward_scalar
import oracle_pins


@pytest.mark.parametrize("name", sorted(oracle_pins.PINS))
def test_pin(name):
    oracle_pins.PINS[name](moda_forward)


def test_pin_brute_force():
    oracle_pins.pin_brute_force(moda_forward, moda_forward_scalar)


def test_rows_subset_matches_full():
    import numpy as np
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 9, 4, 16))
    ks = rng.standard_normal((2, 9, 2, 16))
    vs = rng.standard_normal((2, 9, 2, 16))
    kd = rng.standard_normal((2, 9, 3, 2, 16))
    vd = rng.standard_normal((2, 9, 3, 2, 16))
    out, lse = moda_forward(q, ks, vs, kd, vd)
    rows = [(1, 8, 3), (0, 0, 0), (1, 4, 1), (0, 4, 2)]
    o, l = moda_forward(q, ks, vs, kd, vd, rows=rows)
    for i, (b, t, h) in enumerate(rows):
        assert np.allclose(o[i], out[b, t, h], rtol=0, atol=1e-14)
        assert abs(l[i] - lse[b, h, t]) <= 1e-14
