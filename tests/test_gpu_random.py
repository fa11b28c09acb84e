"""GPU parity on seeded random shapes: the forward over a random depth-slot
window (bf16 or 8-bit depth KV), and for some shapes the backward of that
window (over the same depth KV), each against the oracle.

The shapes are drawn once from a fixed seed (the list is the same on every
run): dtype, head size, kv heads, GQA group size, batch, sequence length
(log-uniform 1..900, so ragged tails and T < one tile both occur), depth
capacity 0..40 and a window [lo, hi) inside it.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_check import TOL, np32
from moda_inputs import make_dout, make_inputs
from oracle import moda_backward, moda_forward
from oracle.moda_quant import dequantize_rows, quantize_rows

pytestmark = pytest.mark.gpu

# max |gpu - oracle| / max(1, max |oracle|) per gradient (as in test_gpu_bwd)
TOL_BWD = {torch.float32: 1e-5, torch.bfloat16: 1.5e-2}


def _draw_cases(n=28, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ("bf16", "fp32")[int(rng.integers(0, 2))]
        d = (64, 128)[int(rng.integers(0, 2))]
        Hkv = int(rng.integers(1, 5))
        G = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32]))
        B = int(rng.integers(1, 3))
        T = int(np.exp(rng.uniform(0.0, np.log(900.0))))
        L_cap = int(rng.integers(0, 41))
        lo = int(rng.integers(0, L_cap + 1))
        hi = int(rng.integers(lo, L_cap + 1))
        q8 = bool(rng.integers(0, 3) == 0) and hi > lo
        bwd = bool(rng.integers(0, 3) == 0)
        cases.append((f"r{i:02d}", dtype, B, T, G * Hkv, Hkv, d, L_cap, lo, hi, q8, bwd))
    return cases


CASES = _draw_cases()


def _say(*a):
    print(*a, flush=True)


def _deq(x):
    codes, scales = quantize_rows(np32(x))
    return dequantize_rows(codes, scales)


@pytest.mark.parametrize("case", CASES, ids=[
    f"{c[0]}_{c[1]}_B{c[2]}_T{c[3]}_Hq{c[4]}_Hkv{c[5]}_d{c[6]}_cap{c[7]}_{c[8]}-{c[9]}"
    f"{'_q8' if c[10] else ''}{'_bwd' if c[11] else ''}" for c in CASES])
def test_random_shape(case):
    name, dtype, B, T, Hq, Hkv, d, L_cap, lo, hi, q8, bwd = case
    _say(f"random case {case}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_cap, dtype=dtype, seed=500 + int(name[1:]))
    dev = torch.device("cuda:0")
    qd, ksd, vsd = q.to(dev), ks.to(dev), vs.to(dev)
    if q8:
        packed = moda.moda_pack_depth_q8(kd.to(dev), vd.to(dev))
        out, lse = moda.moda_fwd_window_q8(qd, ksd, vsd, packed, L_cap, lo, hi)
        kref, vref = _deq(kd)[:, :, lo:hi], _deq(vd)[:, :, lo:hi]
    else:
        kp = vp = None
        if L_cap > 0:
            kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
        out, lse = moda.moda_fwd_window(qd, ksd, vsd, kp, vp, L_cap, lo, hi)
        kref, vref = np32(kd)[:, :, lo:hi], np32(vd)[:, :, lo:hi]
    torch.cuda.synchronize()
    ref_out, ref_lse = moda_forward(np32(q), np32(ks), np32(vs), kref, vref)
    tol = TOL[q.dtype]
    eo = float(np.abs(out.double().cpu().numpy() - ref_out).max())
    el = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
    _say(f"  forward: max|out-ref| = {eo:.3e}  max|lse-ref| = {el:.3e}  (tol {tol:g})")
    assert eo <= tol and el <= tol
    if not bwd:
        return
    dout = make_dout(B, T, Hq, d, dtype=dtype, seed=500 + int(name[1:]))
    if q8:
        grads = moda.moda_bwd_window_q8(qd, ksd, vsd, packed, L_cap, lo, hi, out, lse, dout.to(dev))
    else:
        grads = moda.moda_bwd_window(qd, ksd, vsd, kp, vp, L_cap, lo, hi, out, lse, dout.to(dev))
    torch.cuda.synchronize()
    refs = moda_backward(np32(q), np32(ks), np32(vs), kref, vref, np32(dout))
    tol = TOL_BWD[q.dtype]
    for nm, g, r in zip(("dq", "dk_seq", "dv_seq", "dk_depth", "dv_depth"), grads, refs):
        if r.size == 0:
            continue
        e = float(np.abs(g.double().cpu().numpy() - r).max()) / max(1.0, float(np.abs(r).max()))
        _say(f"  {nm}: {e:.2e}  (tol {tol:g})")
        assert e <= tol, f"{name}: {nm} error {e} > {tol}"
