"""GPU parity of the write step (moda_append_depth) and of depth-slot windows
(moda_fwd_window) against the packed-layout definition and the oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_check import TOL, np32
from moda_inputs import make_inputs
from oracle import moda_forward
from test_gpu_moda import _pack_reference

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _zeros_packed(B, T, Hkv, d, L_cap, dtype):
    n = moda.depth_packed_elems(B, T, Hkv, d, L_cap)
    return (torch.zeros(n, dtype=dtype, device="cuda"), torch.zeros(n, dtype=dtype, device="cuda"))


@pytest.mark.parametrize("case", [("bf16", 2, 37, 3, 128, 5), ("fp32", 1, 64, 2, 64, 3),
                                  ("bf16", 1, 40, 1, 64, 24), ("fp32", 1, 33, 2, 128, 1)])
def test_append_equals_pack(case):
    dtype, B, T, Hkv, d, L = case
    _say(f"append vs pack {case}")
    _, _, _, kd, vd = make_inputs(B, T, Hkv, Hkv, d, L, dtype=dtype, seed=31)
    kp, vp = _zeros_packed(B, T, Hkv, d, L, kd.dtype)
    for j in range(L):
        moda.moda_append_depth(kd[:, :, j].contiguous().cuda(), vd[:, :, j].contiguous().cuda(), kp, vp, L, j)
    kp2, vp2 = moda.moda_pack_depth(kd.cuda(), vd.cuda())
    torch.cuda.synchronize()
    assert torch.equal(kp, kp2) and torch.equal(vp, vp2)
    view = torch.int16 if dtype == "bf16" else torch.int32
    rk, rv = _pack_reference(kd.view(view).numpy(), vd.view(view).numpy())
    assert np.array_equal(kp.cpu().view(view).numpy(), rk)
    assert np.array_equal(vp.cpu().view(view).numpy(), rv)


WINDOWS = [
    # dtype, B, T, Hq, Hkv, d, L_cap, lo, hi
    ("bf16", 1, 300, 8, 2, 128, 6, 2, 5),
    ("bf16", 2, 129, 4, 1, 128, 24, 16, 24),    # sliding window over the last 8 slots
    ("fp32", 1, 100, 4, 2, 64, 5, 0, 0),        # empty window: plain causal attention
    ("fp32", 1, 77, 6, 3, 128, 7, 6, 7),        # one slot
    ("bf16", 1, 1000, 16, 2, 128, 48, 40, 48),  # tiles of one position skipped
    ("bf16", 1, 64, 32, 1, 128, 3, 0, 3),       # whole capacity
    ("bf16", 1, 500, 12, 1, 64, 9, 1, 8),
]


@pytest.mark.parametrize("case", WINDOWS, ids=[f"{c[0]}_T{c[2]}_G{c[3]//c[4]}_cap{c[6]}_{c[7]}-{c[8]}" for c in WINDOWS])
def test_window_parity(case):
    dtype, B, T, Hq, Hkv, d, L_cap, lo, hi = case
    _say(f"window {case}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_cap, dtype=dtype, seed=41 + T)
    dev = torch.device("cuda")
    kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd_window(q.to(dev), ks.to(dev), vs.to(dev), kp, vp, L_cap, lo, hi)
    torch.cuda.synchronize()
    ref_out, ref_lse = moda_forward(np32(q), np32(ks), np32(vs), np32(kd)[:, :, lo:hi], np32(vd)[:, :, lo:hi])
    e_o = float(np.abs(out.double().cpu().numpy() - ref_out).max())
    e_l = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
    tol = TOL[q.dtype]
    _say(f"  max|out-ref| = {e_o:.3e}  max|lse-ref| = {e_l:.3e}  (tol {tol:g})")
    assert e_o <= tol and e_l <= tol


def test_window_of_whole_capacity_is_moda_fwd():
    B, T, Hq, Hkv, d, L = 1, 333, 8, 2, 128, 7
    _say("window [0, L) equals moda_fwd")
    q, ks, vs, kd, vd = [x.cuda() for x in make_inputs(B, T, Hq, Hkv, d, L, dtype="bf16", seed=5)]
    kp, vp = moda.moda_pack_depth(kd, vd)
    o1, l1 = moda.moda_fwd(q, ks, vs, kp, vp, L)
    o2, l2 = moda.moda_fwd_window(q, ks, vs, kp, vp, L, 0, L)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_layer_stack_read_then_write():
    """A 4-layer stack: layer l reads depth slots 0..l-1 (written by the
    layers below) and then appends its own K/V as slot l."""
    B, T, Hq, Hkv, d, L = 1, 200, 8, 2, 128, 4
    _say("layer stack read/write")
    dev = torch.device("cuda")
    kp, vp = _zeros_packed(B, T, Hkv, d, L, torch.bfloat16)
    ks_all, vs_all = [], []
    for layer in range(L):
        q, ks, vs, _, _ = make_inputs(B, T, Hq, Hkv, d, 0, dtype="bf16", seed=100 + layer)
        out, lse = moda.moda_fwd_window(q.to(dev), ks.to(dev), vs.to(dev), kp, vp, L, 0, layer)
        torch.cuda.synchronize()
        if layer:
            kd = np.stack([np32(k) for k in ks_all], axis=2)
            vd = np.stack([np32(v) for v in vs_all], axis=2)
        else:
            kd = np.zeros((B, T, 0, Hkv, d), dtype=np.float32)
            vd = kd
        ref_out, ref_lse = moda_forward(np32(q), np32(ks), np32(vs), kd, vd)
        e_o = float(np.abs(out.double().cpu().numpy() - ref_out).max())
        e_l = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
        _say(f"  layer {layer}: max|out-ref| = {e_o:.3e}  max|lse-ref| = {e_l:.3e}")
        assert e_o <= TOL[torch.bfloat16] and e_l <= TOL[torch.bfloat16]
        moda.moda_append_depth(ks.to(dev), vs.to(dev), kp, vp, L, layer)
        ks_all.append(ks)
        vs_all.append(vs)


def test_window_long_grid_sampled_rows():
    """A window [2, 5) of a 6-slot buffer on a long grid (eight-wave tiles
    from the launch counter, T = 16384, G = 8): sampled rows against the
    oracle on the window's slots."""
    from moda_check import compare_rows
    from moda_inputs import sample_rows
    B, T, Hq, Hkv, d, L_cap, lo, hi = 1, 16384, 16, 2, 128, 6, 2, 5
    _say(f"window on a long grid: B={B} T={T} Hq={Hq} Hkv={Hkv} L_cap={L_cap} window [{lo}, {hi})")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_cap, dtype="bf16", seed=9191)
    dev = torch.device("cuda")
    kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd_window(q.to(dev), ks.to(dev), vs.to(dev), kp, vp, L_cap, lo, hi)
    torch.cuda.synchronize()
    rows = sample_rows(B, T, Hq, n=512, seed=9192, tile_rows=(T - 1, T // 2))
    win = (q, ks, vs, kd[:, :, lo:hi].contiguous(), vd[:, :, lo:hi].contiguous())
    e_o, e_l = compare_rows(win, out.cpu(), lse.cpu(), rows)
    tol = TOL[q.dtype]
    _say(f"  max|out-ref| = {e_o:.3e}  max|lse-ref| = {e_l:.3e}  (tol {tol:g})")
    assert e_o <= tol and e_l <= tol
