"""CPU pins of the backward oracle, and planted mistakes that they must catch."""
import os
import types

import pytest

import oracle_bwd_pins
from oracle import moda_backward, moda_backward_keys

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "moda_backward.py")


@pytest.mark.parametrize("name", sorted(oracle_bwd_pins.BWD_PINS))
def test_backward_pin(name):
    worst = oracle_bwd_pins.BWD_PINS[name](moda_backward)
    print(f"{name}: worst deviation {worst:.3e}")


# Each mutant is a copy of oracle/moda_backward.py with one plausible slip;
# it must fail a pin other than the per-group consistency check.
MUTANTS = {
    "no_jacobian_term": [("dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "dz = p * dp")],
    "jacobian_sign": [("dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                       "dz = p * (dp + (p * dp).sum(axis=1, keepdims=True))")],
    "dq_unscaled": [("dQ = (dz @ Kc) * scale", "dQ = dz @ Kc")],
    "dk_unscaled": [("dK = (dz.T @ Qg) * scale", "dK = dz.T @ Qg")],
    "dk_uses_dout": [("dK = (dz.T @ Qg) * scale", "dK = (dz.T @ dOg) * scale")],
    "dv_unnormalised": [("dV = p.T @ dOg", "dV = e.T @ dOg")],
    "dp_uses_keys": [("dp = dOg @ Vc.T", "dp = dOg @ Kc.T")],
    "depth_grad_prev_position": [("dkd[b, t, :, kvh] = gkd", "dkd[b, max(t - 1, 0), :, kvh] += gkd")],
    "seq_grad_excludes_self": [("dks[b, kvh, : t + 1] += gks", "dks[b, kvh, : t] += gks[:t]")],
    "gqa_first_head_only": [("heads = slice(kvh * G, (kvh + 1) * G)", "heads = slice(kvh * G, kvh * G + 1)")],
    "scale_1_over_d": [("scale = 1.0 / math.sqrt(d)", "scale = 1.0 / d")],
}


def _mutant_module(edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    # the module's relative import of the forward oracle, made absolute
    src = src.replace("from .moda_oracle import moda_forward", "from oracle.moda_oracle import moda_forward")
    mod = types.ModuleType("moda_backward_mutant")
    exec(compile(src, "moda_backward_mutant", "exec"), mod.__dict__)
    return mod


def _mutant(edits):
    return _mutant_module(edits).moda_backward


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_mutant_is_caught(name):
    bwd = _mutant(MUTANTS[name])
    caught = []
    for pname, pin in oracle_bwd_pins.BWD_PINS.items():
        if pname == "groups":
            continue
        try:
            pin(bwd)
        except Exception:
            caught.append(pname)
    assert caught, f"mutant {name} passed every pin"


def test_keys_pin():
    worst = oracle_bwd_pins.pin_keys(moda_backward_keys)
    print(f"keys: worst deviation {worst:.3e}")


# Slips in the per-key form; each must fail the keys pin (the full form it is
# compared with is fixed by finite differences and autograd above).
KEY_MUTANTS = {
    "rows_after_key_only": [("for t in range(s0, T) for h", "for t in range(s0 + 1, T) for h"),
                            ("for t in range(s, T) for h in range(kvh * G", "for t in range(s + 1, T) for h in range(kvh * G"),
                            ("q[b, s:, kvh * G", "q[b, s + 1:, kvh * G"), ("dout[b, s:, kvh * G", "dout[b, s + 1:, kvh * G")],
    "delta_dropped": [("(dOr @ vs_ - delta)", "(dOr @ vs_)")],
    "delta_sign": [("(dOr @ vs_ - delta)", "(dOr @ vs_ + delta)")],
    "key_grad_unscaled": [("@ Qr) * scale", "@ Qr)")],
    "weight_without_lse": [("* scale - lse[idx])", "* scale)")],
    "value_grad_uses_q": [("dv[n] = p @ dOr", "dv[n] = p @ Qr")],
}


@pytest.mark.parametrize("name", sorted(KEY_MUTANTS))
def test_keys_mutant_is_caught(name):
    keys_fn = _mutant_module(KEY_MUTANTS[name]).moda_backward_keys
    with pytest.raises(AssertionError):
        oracle_bwd_pins.pin_keys(keys_fn)
