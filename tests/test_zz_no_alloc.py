"""moda_bwd_noalloc (the backward whose work buffer is the library's static
per-GPU scratch, for callers that cannot allocate) against moda_bwd with a
caller-supplied work buffer, through the C ABI: bit for bit equal gradients,
on two calls in a row, the second with a smaller input."""
from __future__ import annotations

import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_inputs import make_dout, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _case(B, T, Hq, Hkv, d, L_d, dtype, seed):
    print(f"noalloc B{B} T{T} Hq{Hq} Hkv{Hkv} d{d} L{L_d} {dtype}", flush=True)
    q, ks, vs, kd, vd = [x.to(DEV) for x in make_inputs(B, T, Hq, Hkv, d, L_d, dtype=dtype, seed=seed)]
    dout = make_dout(B, T, Hq, d, dtype=dtype, seed=seed).to(DEV)
    kp, vp = moda.moda_pack_depth(kd, vd) if L_d else (None, None)
    out, lse = moda.moda_fwd(q, ks, vs, kp, vp, L_d)
    ref = moda.moda_bwd(q, ks, vs, kp, vp, L_d, out, lse, dout)
    got = tuple(None if g is None else torch.full_like(g, float("nan")) for g in ref)
    moda.moda_bwd_noalloc(q, ks, vs, kp, vp, L_d, out, lse, dout, grads=got)
    torch.cuda.synchronize()
    for r, g in zip(ref, got):
        if r is None:
            assert g is None
        else:
            assert torch.equal(r, g)


def test_noalloc_equals_bwd_two_calls():
    # the second call is smaller: it reuses the scratch the first one left
    _case(2, 700, 16, 2, 128, 6, "bf16", 11)
    _case(1, 90, 4, 1, 64, 3, "fp32", 12)
    _case(1, 300, 8, 2, 128, 0, "bf16", 13)
