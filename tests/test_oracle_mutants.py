"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/moda_oracle.py with one textual change (a
plausible slip: wrong scale, mask off by one, wrong depth position, wrong GQA
map, wrong log base, dropped normalisation, wrong operand, dropped term).  The
copy is executed on the CPU only.  Every mutant must fail at least one pin
other than the scalar brute force (which a shared misreading could also have),
so that the pins, not only the second implementation, constrain the oracle.
"""
import os
import types

import pytest

import oracle_pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moda_oracle.py")

MUTANTS = {
    "scale_1_over_d": [("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d")],
    "no_scale": [("scale = 1.0 / math.sqrt(d)", "scale = 1.0")],
    "causal_excludes_self": [("[b, kvh, : t + 1]", "[b, kvh, : t]"), ("ns = t + 1", "ns = t")],
    "causal_sees_next": [("[b, kvh, : t + 1]", "[b, kvh, : t + 2]"), ("ns = t + 1", "ns = min(t + 2, T)")],
    "depth_prev_position": [("k_depth[b, t, :, kvh, :]", "k_depth[b, max(t - 1, 0), :, kvh, :]")],
    "depth_value_of_prev_position": [("v_depth[b, t, :, kvh, :]", "v_depth[b, max(t - 1, 0), :, kvh, :]")],
    "gqa_interleaved": [("groups[(b, t, kvh)] = list(range(kvh * G, (kvh + 1) * G))",
                         "groups[(b, t, kvh)] = list(range(kvh, Hq, Hkv))")],
    "lse_log2": [("lse = m[:, 0] + np.log(Z[:, 0])", "lse = m[:, 0] + np.log2(Z[:, 0])")],
    "lse_no_max": [("lse = m[:, 0] + np.log(Z[:, 0])", "lse = np.log(Z[:, 0])")],
    "no_normalisation": [("p = e / Z", "p = e / Z.max()")],
    "value_is_key": [("o = p[:, :ns] @ Vs + p[:, ns:] @ Vd", "o = p[:, :ns] @ Ks + p[:, ns:] @ Kd")],
    "depth_values_dropped": [("+ p[:, ns:] @ Vd", "+ 0 * p[:, ns:] @ Vd")],
    "depth_unscaled": [("np.concatenate([Qg @ Ks.T, Qg @ Kd.T], axis=1) * scale",
                        "np.concatenate([(Qg @ Ks.T) * scale, Qg @ Kd.T], axis=1)")],
    "separate_softmax": [("p = e / Z\n", "p = e / Z\n        ns = t + 1\n        p = np.concatenate([e[:, :ns] / e[:, :ns].sum(1, keepdims=True), e[:, ns:] / np.maximum(e[:, ns:].sum(1, keepdims=True), 1e-300)], axis=1) * (0.5 if e.shape[1] > ns else 1.0)\n")],
}


def _mutant(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("moda_oracle_mutant")
    exec(compile(src, "moda_oracle_mutant", "exec"), mod.__dict__)
    return mod.moda_forward


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    fwd = _mutant(MUTANTS[name])
    caught = []
    for pname, pin in oracle_pins.PINS.items():
        try:
            pin(fwd)
        except Exception:
            caught.append(pname)
    assert caught, f"mutant {name} passed every pin"
