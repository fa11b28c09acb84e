"""GPU parity of moda_fwd_ws (the forward with a workspace, whose small grids
split the key range of their longest query tiles over two workgroups) against
the oracle, through the C ABI.

Splitting changes only the order in which the softmax sums are formed (two
partial online-softmax states merged exactly), so every case is held to the
same tolerance as moda_fwd.  The workspace's arrival counters must be back at
zero after every call: repeated calls, and a smaller call after a larger one
on the same workspace, give bit-identical results.
"""
from __future__ import annotations

import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_check import TOL, compare_all_rows, np32
from moda_inputs import make_inputs, workload

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _run_ws(inputs, work=None):
    q, ks, vs, kd, vd = [x.to(DEV) for x in inputs]
    L_d = kd.shape[2]
    kp, vp = moda.moda_pack_depth(kd, vd) if L_d else (None, None)
    if work is None:
        work = moda.fwd_workspace(q, ks)
    out, lse = moda.moda_fwd(q, ks, vs, kp, vp, L_d, work=work)
    torch.cuda.synchronize()
    return out, lse


def _check(name, dtype, err_o, err_l):
    tol = TOL[dtype]
    _say(f"{name}: max|out-ref| = {err_o:.3e}  max|lse-ref| = {err_l:.3e}  (tol {tol:g})")
    assert err_o <= tol and err_l <= tol


def test_split_workload_T4096_all_rows():
    w = workload("bf16_B1_T4096_Hq16_Hkv2_d128_L24")
    B, T, Hq, Hkv, d = w["B"], w["T"], w["Hq"], w["Hkv"], w["d"]
    assert moda.fwd_workspace_bytes(B, T, Hq, Hkv, d, torch.bfloat16) > 0     # this grid splits
    for L_d in (w["L_d"], 0):
        _say(f"split {w['name']} L_d={L_d} (all rows)")
        inputs = make_inputs(B, T, Hq, Hkv, d, L_d, dtype=w["dtype"], seed=w["seed"])
        out, lse = _run_ws(inputs)
        _check(f"{w['name']} L_d={L_d}", inputs[0].dtype, *compare_all_rows(inputs, out, lse))


EDGE = [
    # B, T, Hq, Hkv, L_d (bf16, d = 128); B large enough for two rounds of
    # 128-row tiles (a grid of one round splits inside the workgroup instead)
    (5, 1000, 8, 1, 5),      # G = 8, ragged last tile
    (19, 777, 2, 2, 0),      # G = 1, no depth
    (4, 300, 32, 1, 3),      # G = 32
    (4, 130, 64, 1, 2),      # G = 64: two positions per 128-row tile
    (8, 257, 16, 2, 24),     # odd tile count per (b, kv head)
    (33, 129, 4, 4, 33),     # G = 1, L_d > 32
    (65, 40, 12, 1, 3),      # G = 12, few tiles: the split parts of short tiles
    (1, 1, 8, 2, 3),         # one position: one tile, nothing to split
    (2, 2048, 16, 4, 7),     # G = 4, 8 (b, kv head) x 64 tiles: the largest split grid (512)
]


@pytest.mark.parametrize("case", EDGE, ids=[f"B{c[0]}_T{c[1]}_Hq{c[2]}_Hkv{c[3]}_L{c[4]}" for c in EDGE])
def test_split_edge_shapes(case):
    B, T, Hq, Hkv, L_d = case
    need = moda.fwd_workspace_bytes(B, T, Hq, Hkv, 128, torch.bfloat16)
    assert need > 0 or T == 1
    _say(f"split edge {case} (workspace {need} bytes)")
    inputs = make_inputs(B, T, Hq, Hkv, 128, L_d, dtype="bf16", seed=90 + T + L_d)
    out, lse = _run_ws(inputs)
    _check(str(case), inputs[0].dtype, *compare_all_rows(inputs, out, lse))


def test_split_repeated_calls_agree():
    """Counters return to zero: the same call twice, then a smaller grid, then
    the first call again, all on one workspace, give bit-identical results;
    and the split result agrees with moda_fwd within the tolerance."""
    big = make_inputs(1, 4096, 16, 2, 128, 24, dtype="bf16", seed=5)
    small = make_inputs(2, 700, 8, 1, 128, 3, dtype="bf16", seed=6)
    q = big[0].to(DEV)
    ks = big[1].to(DEV)
    work = moda.fwd_workspace(q, ks)
    _say("split: repeated calls on one workspace")
    o1, l1 = _run_ws(big, work)
    o2, l2 = _run_ws(big, work)
    s1, t1 = _run_ws(small, work)
    o3, l3 = _run_ws(big, work)
    s2, t2 = _run_ws(small, work)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)
    assert torch.equal(s1, s2) and torch.equal(t1, t2)
    # every counter (the 4096-byte header) is back at zero
    assert int(work[:4096].view(torch.int32).abs().sum()) == 0
    # a second input set of the same shape on the same workspace, alternating
    # with the first: each result equals the one from a fresh workspace (a
    # merge that read the other call's partial state would not)
    big2 = make_inputs(1, 4096, 16, 2, 128, 24, dtype="bf16", seed=7)
    r2, q2 = _run_ws(big2)
    for _ in range(3):
        a1, b1 = _run_ws(big, work)
        a2, b2 = _run_ws(big2, work)
        assert torch.equal(a1, o1) and torch.equal(b1, l1)
        assert torch.equal(a2, r2) and torch.equal(b2, q2)
    # against the unsplit forward on the same inputs
    kp, vp = moda.moda_pack_depth(big[3].to(DEV), big[4].to(DEV))
    o0, l0 = moda.moda_fwd(q, ks, big[2].to(DEV), kp, vp, 24)
    torch.cuda.synchronize()
    tol = TOL[torch.bfloat16]
    assert float((o0.float() - o1.float()).abs().max()) <= tol
    assert float((l0 - l1).abs().max()) <= tol
    assert np32(o1).shape == (1, 4096, 16, 128)


def test_one_round_grid_needs_no_workspace():
    """A grid that fits one round of eight-wave workgroups splits each tile's
    keys inside the workgroup: no workspace, and moda_fwd_ws gives moda_fwd's
    results bit for bit."""
    B, T, Hq, Hkv, L_d = 1, 1000, 8, 1, 5
    assert moda.fwd_workspace_bytes(B, T, Hq, Hkv, 128, torch.bfloat16) == 0
    _say("one-round grid: moda_fwd_ws == moda_fwd")
    q, ks, vs, kd, vd = [x.cuda() for x in make_inputs(B, T, Hq, Hkv, 128, L_d, dtype="bf16", seed=77)]
    packed = moda.moda_pack_depth(kd, vd)
    o1, l1 = moda.moda_fwd(q, ks, vs, *packed, L_d)
    o2, l2 = moda.moda_fwd(q, ks, vs, *packed, L_d, work=moda.fwd_workspace(q, ks))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
