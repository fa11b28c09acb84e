"""CPU pins of the 8-bit depth-KV oracle (oracle/moda_quant.py)."""
import numpy as np
import pytest

from oracle import moda_forward
from oracle.moda_quant import dequantize_rows, quantize_rows, quantize_rows_scalar


def _rows(seed, n=64, d=128, dist="normal"):
    rng = np.random.default_rng(seed)
    if dist == "normal":
        return rng.standard_normal((n, d)).astype(np.float32)
    return (rng.standard_cauchy((n, d)) * 0.1).astype(np.float32)


@pytest.mark.parametrize("dist", ["normal", "heavy"])
def test_rounding_bound_and_range(dist):
    x = _rows(1, dist=dist)
    q, s = quantize_rows(x)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.abs(q.astype(int)).max() <= 127
    err = np.abs(x.astype(np.float64) - dequantize_rows(q, s))
    # |x - s*code| <= s/2 up to the float32 rounding of x/s (a few ulps of the quotient)
    assert np.all(err <= s[:, None].astype(np.float64) * (0.5 + 1e-5))


def test_row_max_maps_to_127():
    x = _rows(2)
    q, s = quantize_rows(x)
    i = np.argmax(np.abs(x), axis=1)
    top = q[np.arange(len(x)), i].astype(int)
    assert np.all(np.abs(top) == 127)
    assert np.all(np.sign(top) == np.sign(x[np.arange(len(x)), i]))


def test_exact_codes_for_integer_rows():
    # rows k * 2^-e with max |k| = 127 quantise exactly: scale = 2^-e
    rng = np.random.default_rng(3)
    k = rng.integers(-127, 128, size=(16, 64))
    k[:, 0] = 127
    x = (k * 2.0 ** -5).astype(np.float32)
    q, s = quantize_rows(x)
    assert np.all(s == np.float32(2.0 ** -5))
    assert np.array_equal(q.astype(int), k)
    assert np.array_equal(dequantize_rows(q, s), x.astype(np.float64))


def test_sign_symmetry_and_zero_row():
    x = _rows(4)
    x[5] = 0.0
    q, s = quantize_rows(x)
    qn, sn = quantize_rows(-x)
    assert np.array_equal(s, sn) and np.array_equal(q.astype(int), -qn.astype(int))
    assert s[5] == 0 and not q[5].any()


def test_scalar_implementation_agrees_bitwise():
    for seed, dist in ((5, "normal"), (6, "heavy")):
        x = _rows(seed, n=24, d=32, dist=dist)
        q, s = quantize_rows(x)
        qs, ss = quantize_rows_scalar(x)
        assert np.array_equal(q.astype(int), np.array(qs))
        assert np.array_equal(s, np.array(ss, dtype=np.float32))


def test_ties_round_to_even():
    # x / scale lands exactly on .5: codes round to even
    x = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.0]], dtype=np.float32)
    q, s = quantize_rows(x)
    assert s[0] == np.float32(1.0)
    assert q[0].tolist() == [127, 0, 2, 2, 0, -2, -2, 3]


def test_quantised_forward_is_forward_of_dequantised_depth():
    """The quantised MoDA forward is the plain forward on the dequantised depth
    KV; with codes that represent the inputs exactly it equals the forward on
    the inputs themselves."""
    rng = np.random.default_rng(7)
    B, T, Hq, Hkv, d, L = 1, 6, 4, 2, 8, 3
    q = rng.standard_normal((B, T, Hq, d))
    ks = rng.standard_normal((B, T, Hkv, d))
    vs = rng.standard_normal((B, T, Hkv, d))
    k = rng.integers(-127, 128, size=(B, T, L, Hkv, d))
    k[..., 0] = 127
    kd = (k * 2.0 ** -6).astype(np.float32)
    vd = (np.roll(k, 1, axis=-1) * 2.0 ** -4).astype(np.float32)
    kq, ksc = quantize_rows(kd)
    vq, vsc = quantize_rows(vd)
    o1, l1 = moda_forward(q, ks, vs, dequantize_rows(kq, ksc), dequantize_rows(vq, vsc))
    o2, l2 = moda_forward(q, ks, vs, kd, vd)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# Planted mistakes in quantize_rows; each must fail a pin other than the
# scalar cross-check (which could share a misreading).
import os
import types

_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moda_quant.py")
_MUTANTS = {
    "scale_over_128": [("absmax / np.float32(127.0)", "absmax / np.float32(128.0)")],
    "floor_not_rint": [("r = np.rint(x32 / safe[..., None])", "r = np.floor(x32 / safe[..., None])")],
    "ties_away": [("r = np.rint(x32 / safe[..., None])", "r = np.trunc(x32 / safe[..., None] + np.sign(x32) * 0.5)")],
    "mean_abs_scale": [("absmax = np.max(np.abs(x32), axis=-1)", "absmax = np.mean(np.abs(x32), axis=-1) * 3")],
    "no_clamp_uint": [("r = np.clip(r, -127, 127)", "r = np.clip(r, 0, 127)")],
    "dequant_no_scale": [("return np.asarray(scales, dtype=np.float64)[..., None] * np.asarray(codes, dtype=np.float64)",
                          "return np.asarray(codes, dtype=np.float64) / 127.0")],
}


def _mutant(edits):
    src = open(_SRC).read()
    for old, new in edits:
        assert old in src, old
        src = src.replace(old, new)
    mod = types.ModuleType("moda_quant_mutant")
    exec(compile(src, "moda_quant_mutant", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(_MUTANTS))
def test_quant_mutant_is_caught(name, monkeypatch):
    import sys
    m = _mutant(_MUTANTS[name])
    mod = sys.modules[__name__]
    monkeypatch.setattr(mod, "quantize_rows", m.quantize_rows)
    monkeypatch.setattr(mod, "dequantize_rows", m.dequantize_rows)
    pins = [lambda: test_rounding_bound_and_range("normal"), lambda: test_rounding_bound_and_range("heavy"),
            test_row_max_maps_to_127, test_exact_codes_for_integer_rows, test_sign_symmetry_and_zero_row,
            test_ties_round_to_even, test_quantised_forward_is_forward_of_dequantised_depth]
    failed = 0
    for pin in pins:
        try:
            pin()
        except Exception:
            failed += 1
    assert failed, f"mutant {name} passed every pin"
