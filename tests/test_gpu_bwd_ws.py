"""GPU parity of moda_bwd_ws (the backward whose dK/dV rows are split over
several workgroups on short sequences, through the C ABI) against the
float64 backward oracle, and against moda_bwd.

The split changes only the order in which dk and dv are summed, so the
bound on the error against the oracle is moda_bwd's; the results must also be
the same from call to call (the partial sums are added in a fixed order),
whatever the workspace held before.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_check import key_errors, np32, rel_err, tail_keys
from moda_inputs import make_dout, make_inputs, workload
from oracle import moda_backward

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
TOL_BWD = {torch.float32: 1e-5, torch.bfloat16: 1.5e-2}   # as for moda_bwd
NAMES = ("dq", "dk_seq", "dv_seq", "dk_depth", "dv_depth")


def _say(*a):
    print(*a, flush=True)


def _work_bytes(B, T, Hq):
    return (2 * B * Hq * T * 4 + 255) // 256 * 256


def _fwd(q, ks, vs, kd, vd):
    L_d = kd.shape[2]
    qd, ksd, vsd = q.to(DEV), ks.to(DEV), vs.to(DEV)
    kp = vp = None
    if L_d > 0:
        kp, vp = moda.moda_pack_depth(kd.to(DEV), vd.to(DEV))
    out, lse = moda.moda_fwd(qd, ksd, vsd, kp, vp, L_d)
    return qd, ksd, vsd, kp, vp, L_d, out, lse


def _bwd_ws(qd, ksd, vsd, kp, vp, L_d, out, lse, dd, fill):
    ws = moda.bwd_workspace(qd, ksd)
    ws.fill_(fill)                                 # stale contents: every byte read must be written first
    g = moda.moda_bwd(qd, ksd, vsd, kp, vp, L_d, out, lse, dd, workspace=ws)
    torch.cuda.synchronize()
    return g


def _np(grads, B, T, Hkv, d):
    got = [None if g is None else g.double().cpu().numpy() for g in grads]
    if got[3] is None:
        got[3] = got[4] = np.zeros((B, T, 0, Hkv, d))
    return got


CASES = [
    # name, dtype, B, T, Hq, Hkv, d, L_d, splits
    ("bf16_T1000_G8_L3", "bf16", 1, 1000, 8, 1, 128, 3, True),
    ("bf16_B2_T700_G6_L4", "bf16", 2, 700, 12, 2, 128, 4, True),     # G not dividing 64
    ("bf16_T2000_G1_L0", "bf16", 1, 2000, 2, 2, 128, 0, True),
    ("bf16_T257_G64_L2", "bf16", 1, 257, 64, 1, 128, 2, True),
    ("bf16_B3_T333_G5_L2", "bf16", 3, 333, 10, 2, 128, 2, True),
    ("bf16_T300_G16_L5", "bf16", 1, 300, 16, 1, 128, 5, True),
    ("bf16_T200_G8_L2", "bf16", 1, 200, 8, 1, 128, 2, True),        # two key tiles
    ("bf16_T1025_G8_L4", "bf16", 1, 1025, 8, 1, 128, 4, True),      # last key tile one key long
    ("bf16_B2_T1500_G2_L3", "bf16", 2, 1500, 4, 2, 128, 3, True),
    ("bf16_T3000_G8_L6", "bf16", 1, 3000, 24, 3, 128, 6, True),     # three kv heads, ragged tail
    ("bf16_T512_G2_L3", "bf16", 1, 512, 8, 4, 128, 3, False),       # 16 query blocks: too few to cut
    ("bf16_T100_G8_L3", "bf16", 1, 100, 8, 1, 128, 3, False),       # one key tile
    ("fp32_T200_G4_d64_L2", "fp32", 1, 200, 4, 1, 64, 2, False),    # generic kernels: as moda_bwd
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_ws_parity(case):
    name, dtype, B, T, Hq, Hkv, d, L_d, splits = case
    _say(f"bwd_ws {name}")
    seed = 300 + T + Hq
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype=dtype, seed=seed)
    dout = make_dout(B, T, Hq, d, dtype=dtype, seed=seed)
    need = moda.bwd_workspace_bytes(B, T, Hq, Hkv, d, q.dtype)
    assert (need > _work_bytes(B, T, Hq)) == splits, (need, _work_bytes(B, T, Hq))
    args = _fwd(q, ks, vs, kd, vd)
    dd = dout.to(DEV)
    g1 = _bwd_ws(*args, dd, 255)                   # NaN bit patterns in the workspace
    g2 = _bwd_ws(*args, dd, 0)
    for a, b in zip(g1, g2):
        assert (a is None) == (b is None)
        if a is not None:
            assert torch.equal(a, b), "moda_bwd_ws differs between calls"
    got = _np(g1, B, T, Hkv, d)
    ref = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout))
    tol = TOL_BWD[q.dtype]
    errs = {nm: rel_err(got[i], ref[i]) for i, nm in enumerate(NAMES) if ref[i].size}
    _say(f"{name}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{name}: {k} error {v} > {tol}"
    # against moda_bwd: dq and the depth gradients come from the same kernels;
    # without a split every gradient is moda_bwd's
    base = moda.moda_bwd(*args, dd)
    torch.cuda.synchronize()
    for i in ((0, 3, 4) if splits else (0, 1, 2, 3, 4)):
        if base[i] is not None:
            assert torch.equal(base[i], g1[i]), f"{NAMES[i]} differs from moda_bwd"


def test_bwd_ws_workload_T4096_all_elements():
    w = workload("bf16_B1_T4096_Hq16_Hkv2_d128_L24")
    B, T, Hq, Hkv, d, L_d = w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"]
    _say(f"bwd_ws {w['name']} (all elements)")
    assert moda.bwd_workspace_bytes(B, T, Hq, Hkv, d, torch.bfloat16) > _work_bytes(B, T, Hq)
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype=w["dtype"], seed=w["seed"])
    dout = make_dout(B, T, Hq, d, dtype=w["dtype"], seed=w["seed"])
    args = _fwd(q, ks, vs, kd, vd)
    dd = dout.to(DEV)
    g1 = _bwd_ws(*args, dd, 255)
    g2 = _bwd_ws(*args, dd, 7)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b), "moda_bwd_ws differs between calls"
    got = _np(g1, B, T, Hkv, d)
    ref = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout))
    tol = TOL_BWD[torch.bfloat16]
    errs = {nm: rel_err(got[i], ref[i]) for i, nm in enumerate(NAMES)}
    _say(f"{w['name']} ws: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{k} error {v} > {tol}"


def test_bwd_ws_T16384_B1_sampled_keys():
    """B = 1, T = 16384 (128 key tiles per kv head, the first swept by a dozen
    chunks): the sequence-key gradients of the first two key tiles, of keys
    around chunk-length boundaries and of the last keys against the oracle's
    per-key form, and the exact sums (sum of dv = sum of dout, sum of dk = 0)."""
    B, T, Hq, Hkv, d, L_d = 1, 16384, 16, 2, 128, 24
    _say(f"bwd_ws B{B} T{T} Hq{Hq} Hkv{Hkv} d{d} L{L_d} (sampled keys + gradient sums)")
    assert moda.bwd_workspace_bytes(B, T, Hq, Hkv, d, torch.bfloat16) > _work_bytes(B, T, Hq)
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype="bf16", seed=91)
    dout = make_dout(B, T, Hq, d, dtype="bf16", seed=91)
    args = _fwd(q, ks, vs, kd, vd)
    dq, dks, dvs, dkd, dvd = _bwd_ws(*args, dout.to(DEV), 255)
    keys = sorted(set(range(0, 256, 3)) | {255, 1023, 1024, 4095, 4096, 8191, 8192} | set(tail_keys(T)))
    errs = key_errors("ws", np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), dks, dvs, B, Hkv, keys)
    G = Hq // Hkv
    do = np32(dout).astype(np.float64)
    dks_, dvs_ = dks.double().cpu().numpy(), dvs.double().cpu().numpy()
    dkd_, dvd_ = dkd.double().cpu().numpy(), dvd.double().cpu().numpy()
    for kvh in range(Hkv):
        sv = dvs_[0, :, kvh].sum(0) + dvd_[0, :, :, kvh].sum((0, 1))
        ref = do[0, :, kvh * G:(kvh + 1) * G].sum((0, 1))
        l1v = np.abs(dvs_[0, :, kvh]).sum(0) + np.abs(dvd_[0, :, :, kvh]).sum((0, 1))
        sk = dks_[0, :, kvh].sum(0) + dkd_[0, :, :, kvh].sum((0, 1))
        l1k = np.abs(dks_[0, :, kvh]).sum(0) + np.abs(dkd_[0, :, :, kvh]).sum((0, 1))
        errs[f"sum_dv[{kvh}]"] = float((np.abs(sv - ref) / l1v).max())
        errs[f"sum_dk[{kvh}]"] = float((np.abs(sk) / l1k).max())
    tol = TOL_BWD[torch.bfloat16]
    _say("T16384 ws: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{k} error {v} > {tol}"


def test_bwd_ws_rejects_small_workspace():
    B, T, Hq, Hkv, d = 1, 1000, 8, 1, 128
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, 2, dtype="bf16", seed=5)
    args = _fwd(q, ks, vs, kd, vd)
    need = moda.bwd_workspace_bytes(B, T, Hq, Hkv, d, torch.bfloat16)
    ws = torch.empty(need - 256, dtype=torch.uint8, device=DEV)
    with pytest.raises(moda.ModaError):
        moda.moda_bwd(*args, make_dout(B, T, Hq, d, dtype="bf16", seed=5).to(DEV), workspace=ws)
