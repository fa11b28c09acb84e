"""GPU parity of the backward (moda_bwd, through the C ABI) against the
float64 backward oracle on the same seeded inputs.

The forward that feeds it is the GPU forward (as in training: the backward
consumes that forward's out and lse).  Each gradient is compared element by
element; the error is measured relative to max(1, max |reference|) of that
gradient, since sums over many rows (dk, dv of early keys) grow with T.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_check import key_errors, np32, rel_err as _rel_err, tail_keys
from moda_inputs import make_dout, make_inputs, workload
from oracle import moda_backward

pytestmark = pytest.mark.gpu

# Bounds on max|gpu - oracle| / max(1, max|oracle|), per gradient.  float32:
# float32 products end to end.  bf16: P and dS enter the matrix-core products
# rounded to bf16 (relative 2^-9 each) and every gradient is rounded to bf16
# on output (relative 2^-9), the same error budget as the forward's 1.5e-2.
TOL_BWD = {torch.float32: 1e-5, torch.bfloat16: 1.5e-2}
NAMES = ("dq", "dk_seq", "dv_seq", "dk_depth", "dv_depth")


def _say(*a):
    print(*a, flush=True)


def run_fwd_bwd(q, ks, vs, kd, vd, dout):
    dev = torch.device("cuda:0")
    L_d = kd.shape[2]
    qd, kd_, vd_, dd = q.to(dev), ks.to(dev), vs.to(dev), dout.to(dev)
    kp = vp = None
    if L_d > 0:
        kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd(qd, kd_, vd_, kp, vp, L_d)
    grads = moda.moda_bwd(qd, kd_, vd_, kp, vp, L_d, out, lse, dd)
    torch.cuda.synchronize()
    return [None if g is None else g.double().cpu().numpy() for g in grads]


def _check_all(name, dtype, got, ref):
    tol = TOL_BWD[dtype]
    errs = {}
    for i, nm in enumerate(NAMES):
        if ref[i].size == 0:
            continue
        errs[nm] = _rel_err(got[i], ref[i])
    _say(f"{name}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{name}: {k} error {v} > {tol}"


CASES = [
    # name, dtype, B, T, Hq, Hkv, d, L_d
    ("fp32_B1_T128_Hq4_Hkv1_d64_L3", "fp32", 1, 128, 4, 1, 64, 3),
    ("bf16_T300_G4_d128_L5", "bf16", 1, 300, 8, 2, 128, 5),
    ("bf16_B2_T97_G3_d128_L4", "bf16", 2, 97, 6, 2, 128, 4),
    ("bf16_T64_G1_d64_L2", "bf16", 1, 64, 2, 2, 64, 2),
    ("fp32_T77_G2_d128_L2", "fp32", 1, 77, 4, 2, 128, 2),
    ("fp32_T150_G3_d64_L7", "fp32", 1, 150, 3, 1, 64, 7),
    ("bf16_T130_G32_d128_L6", "bf16", 1, 130, 32, 1, 128, 6),
    ("bf16_T200_G4_d128_L0", "bf16", 1, 200, 4, 1, 128, 0),
    ("bf16_T1_G2_d128_L3", "bf16", 1, 1, 4, 2, 128, 3),
    ("bf16_T257_G8_d128_L40", "bf16", 1, 257, 16, 2, 128, 40),
    # G dividing 64 (dK/dV rows addressed from each block's base) and not
    ("bf16_B2_T150_G1_d128_L3", "bf16", 2, 150, 2, 2, 128, 3),
    ("bf16_T100_G64_d128_L2", "bf16", 1, 100, 64, 1, 128, 2),
    ("bf16_T70_G16_d128_L5", "bf16", 1, 70, 32, 2, 128, 5),
    ("bf16_T90_G12_d128_L3", "bf16", 1, 90, 12, 1, 128, 3),
    ("bf16_T33_G5_d128_L0", "bf16", 1, 33, 5, 1, 128, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(case):
    name, dtype, B, T, Hq, Hkv, d, L_d = case
    _say(f"bwd {name}")
    seed = 60 + T + Hq
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype=dtype, seed=seed)
    dout = make_dout(B, T, Hq, d, dtype=dtype, seed=seed)
    got = run_fwd_bwd(q, ks, vs, kd, vd, dout)
    ref = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout))
    if L_d == 0:
        assert got[3] is None and got[4] is None
        got = got[:3] + [np.zeros((B, T, 0, Hkv, d))] * 2
    _check_all(name, q.dtype, got, ref)


def test_bwd_workload_T4096_all_elements():
    w = workload("bf16_B1_T4096_Hq16_Hkv2_d128_L24")
    _say(f"bwd {w['name']} (all elements)")
    q, ks, vs, kd, vd = make_inputs(w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"],
                                    dtype=w["dtype"], seed=w["seed"])
    dout = make_dout(w["B"], w["T"], w["Hq"], w["d"], dtype=w["dtype"], seed=w["seed"])
    got = run_fwd_bwd(q, ks, vs, kd, vd, dout)
    ref = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout))
    _check_all(w["name"], q.dtype, got, ref)


@pytest.mark.parametrize("name", ["bf16_B2_T16384_Hq16_Hkv2_d128_L24", "bf16_B1_T65536_Hq16_Hkv2_d128_L24",
                                  "bf16_B1_T65536_Hq32_Hkv1_d128_L48"])
def test_bwd_workload_sampled(name):
    """At the 16K and 64K workloads: the query and depth-slot gradients of
    sampled (b, t, kv head) groups against the oracle's per-group form, the
    sequence-key gradients of the last keys and of the keys around the last
    128-key tile boundaries against its per-key form (every batch and kv
    head), and the exact sums (sum of dv over all keys = sum of dout; sum of
    dk = 0) per (batch, kv head)."""
    w = workload(name)
    _say(f"bwd {w['name']} (sampled groups + gradient sums)")
    B, T, Hq, Hkv, d, L_d = w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"]
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype=w["dtype"], seed=w["seed"])
    dout = make_dout(B, T, Hq, d, dtype=w["dtype"], seed=w["seed"])
    dq, dks, dvs, dkd, dvd = run_fwd_bwd(q, ks, vs, kd, vd, dout)
    G = Hq // Hkv
    rng = np.random.default_rng(w["seed"] + 11)
    ts = sorted(set(rng.integers(0, T, 40).tolist()) | {0, 1, 63, 64, T // 2, T - 1})
    groups = [(int(rng.integers(0, B)) if B > 1 else 0, t, kvh) for t in ts for kvh in range(Hkv)]
    groups += [(B - 1, T - 1, kvh) for kvh in range(Hkv)] if B > 1 else []
    rq, rkd, rvd = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), groups=groups)
    gq = np.stack([dq[b, t, kvh * G:(kvh + 1) * G] for (b, t, kvh) in groups])
    gkd = np.stack([dkd[b, t, :, kvh] for (b, t, kvh) in groups])
    gvd = np.stack([dvd[b, t, :, kvh] for (b, t, kvh) in groups])
    tol = TOL_BWD[q.dtype]
    errs = {"dq": _rel_err(gq, rq), "dk_depth": _rel_err(gkd, rkd), "dv_depth": _rel_err(gvd, rvd)}
    # sequence-key gradients element by element at the last keys (both batches)
    errs.update(key_errors("tail", np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), dks, dvs, B, Hkv,
                           tail_keys(T)))
    # exact sums, checked relative to the L1 size of the summands
    do = np32(dout).astype(np.float64)
    for b in range(B):
        for kvh in range(Hkv):
            sv = dvs[b, :, kvh].sum(0) + dvd[b, :, :, kvh].sum((0, 1))
            ref = do[b, :, kvh * G:(kvh + 1) * G].sum((0, 1))
            l1v = np.abs(dvs[b, :, kvh]).sum(0) + np.abs(dvd[b, :, :, kvh]).sum((0, 1))
            sk = dks[b, :, kvh].sum(0) + dkd[b, :, :, kvh].sum((0, 1))
            l1k = np.abs(dks[b, :, kvh]).sum(0) + np.abs(dkd[b, :, :, kvh]).sum((0, 1))
            errs[f"sum_dv[{b},{kvh}]"] = float((np.abs(sv - ref) / l1v).max())
            errs[f"sum_dk[{b},{kvh}]"] = float((np.abs(sk) / l1k).max())
    _say(f"{w['name']}: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{k} error {v} > {tol}"


def test_bwd_long_sequence():
    """T * Hq * d * 2 bytes = 2^31 (past 32-bit byte offsets from the batch's
    first row; G = 32 divides the 64-row blocks, so the dK/dV kernel addresses
    rows from each block's base): sampled groups against the oracle, the last
    sequence keys element by element, and the exact gradient sums."""
    B, T, Hq, Hkv, d, L_d = 1, 262144, 32, 1, 128, 2
    _say(f"bwd long sequence B{B} T{T} Hq{Hq} Hkv{Hkv} d{d} L{L_d}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype="bf16", seed=77)
    dout = make_dout(B, T, Hq, d, dtype="bf16", seed=77)
    dev = torch.device("cuda:0")
    qd, ksd, vsd, dd = q.to(dev), ks.to(dev), vs.to(dev), dout.to(dev)
    kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd(qd, ksd, vsd, kp, vp, L_d)
    dq, dks, dvs, dkd, dvd = moda.moda_bwd(qd, ksd, vsd, kp, vp, L_d, out, lse, dd)
    torch.cuda.synchronize()
    del out, lse, kp, vp
    G = Hq // Hkv
    rng = np.random.default_rng(78)
    ts = sorted(set(rng.integers(0, T, 6).tolist()) | {0, 1, 63, 64, T // 2, T - 1})
    groups = [(0, t, 0) for t in ts]
    rq, rkd, rvd = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), groups=groups)
    idx = torch.tensor(ts, device=dev)
    gq = dq[0].index_select(0, idx).double().cpu().numpy()            # [n, Hq, d]
    gkd = dkd[0].index_select(0, idx)[:, :, 0].double().cpu().numpy()  # [n, L_d, d]
    gvd = dvd[0].index_select(0, idx)[:, :, 0].double().cpu().numpy()
    errs = {"dq": _rel_err(gq, rq), "dk_depth": _rel_err(gkd, rkd), "dv_depth": _rel_err(gvd, rvd)}
    # the last keys (highest q / dO offsets of the dK/dV kernel) element by element
    errs.update(key_errors("tail", np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), dks, dvs, B, Hkv,
                           tail_keys(T, last=32, bounds=(128,))))
    dvs_, dks_ = dvs[0, :, 0].double().cpu().numpy(), dks[0, :, 0].double().cpu().numpy()
    dvd_, dkd_ = dvd[0, :, :, 0].double().cpu().numpy(), dkd[0, :, :, 0].double().cpu().numpy()
    ref = dout[0].sum((0, 1), dtype=torch.float64).numpy()
    sv = dvs_.sum(0) + dvd_.sum((0, 1))
    sk = dks_.sum(0) + dkd_.sum((0, 1))
    errs["sum_dv"] = float((np.abs(sv - ref) / (np.abs(dvs_).sum(0) + np.abs(dvd_).sum((0, 1)))).max())
    errs["sum_dk"] = float((np.abs(sk) / (np.abs(dks_).sum(0) + np.abs(dkd_).sum((0, 1)))).max())
    tol = TOL_BWD[torch.bfloat16]
    _say("long sequence: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{k} error {v} > {tol}"


@pytest.mark.parametrize("case", [("bf16", 1, 180, 8, 2, 128, 6, 2, 5), ("fp32", 1, 70, 4, 1, 64, 5, 3, 5),
                                  ("bf16", 1, 100, 6, 2, 128, 4, 0, 4)])
def test_bwd_window_parity(case):
    """Backward of a depth-slot window: the oracle backward of the forward over
    the window's slots; depth gradients are those of the window's slots."""
    dtype, B, T, Hq, Hkv, d, L_cap, lo, hi = case
    _say(f"bwd window {case}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_cap, dtype=dtype, seed=80 + T)
    dout = make_dout(B, T, Hq, d, dtype=dtype, seed=80 + T)
    dev = torch.device("cuda:0")
    kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
    qd, ksd, vsd, dd = q.to(dev), ks.to(dev), vs.to(dev), dout.to(dev)
    out, lse = moda.moda_fwd_window(qd, ksd, vsd, kp, vp, L_cap, lo, hi)
    grads = moda.moda_bwd_window(qd, ksd, vsd, kp, vp, L_cap, lo, hi, out, lse, dd)
    torch.cuda.synchronize()
    got = [g.double().cpu().numpy() for g in grads]
    ref = moda_backward(np32(q), np32(ks), np32(vs), np32(kd)[:, :, lo:hi], np32(vd)[:, :, lo:hi], np32(dout))
    _check_all(f"window {case}", q.dtype, got, ref)


def test_bwd_counter_order_repeatable_and_concurrent():
    """With B * Hkv <= 2 the long dQ and dK/dV grids take their tiles from
    per-launch counter slots that each launch returns to zero: backward calls
    in a row, and calls in flight at the same time on two streams, give
    bit-identical gradients (a slot left non-zero would make the next launch
    skip tiles)."""
    B, T, Hq, Hkv, d, L = 1, 32768, 16, 2, 128, 4
    _say(f"bwd counter order: B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} L_d={L} (dQ 4096 and dK/dV 512 workgroups)")
    dev = torch.device("cuda:0")
    q, ks, vs, kd, vd = [x.to(dev) for x in make_inputs(B, T, Hq, Hkv, d, L, dtype="bf16", seed=5151)]
    dout = make_dout(B, T, Hq, d, dtype="bf16", seed=5152).to(dev)
    kp, vp = moda.moda_pack_depth(kd, vd)
    out, lse = moda.moda_fwd(q, ks, vs, kp, vp, L)
    ref = moda.moda_bwd(q, ks, vs, kp, vp, L, out, lse, dout)
    runs = [moda.moda_bwd(q, ks, vs, kp, vp, L, out, lse, dout)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for s in (s1, s2):
        g = tuple(torch.empty_like(x) for x in ref)
        w = torch.empty(2, B, Hq, T, dtype=torch.float32, device=dev)
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            moda.moda_bwd(q, ks, vs, kp, vp, L, out, lse, dout, grads=g, work=w, stream=s)
        runs.append(g)
    torch.cuda.synchronize()
    for i, g in enumerate(runs):
        for name, a, b in zip(NAMES, ref, g):
            assert torch.equal(a, b), f"call {i + 1}: {name} differs from the first call"


def test_bwd_counter_nine_pairs():
    """Nine (b, kv head) pairs (B = 3, Hkv = 3): the dQ and dK/dV grids
    (1152 and 576 workgroups) take their tiles from nine per-pair queues,
    workgroups moving on to the following pairs' queues once their own is
    empty.  Sampled query groups, the last keys of every pair and the exact
    gradient sums against the oracle; a second call bit-equal to the first."""
    B, T, Hq, Hkv, d, L_d = 3, 8192, 6, 3, 128, 3
    _say(f"bwd nine pairs: B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} L_d={L_d}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype="bf16", seed=6161)
    dout = make_dout(B, T, Hq, d, dtype="bf16", seed=6162)
    dev = torch.device("cuda:0")
    qd, ksd, vsd, dd = q.to(dev), ks.to(dev), vs.to(dev), dout.to(dev)
    kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd(qd, ksd, vsd, kp, vp, L_d)
    g1 = moda.moda_bwd(qd, ksd, vsd, kp, vp, L_d, out, lse, dd)
    g2 = moda.moda_bwd(qd, ksd, vsd, kp, vp, L_d, out, lse, dd)
    torch.cuda.synchronize()
    for name, a, b in zip(NAMES, g1, g2):
        assert torch.equal(a, b), f"second call: {name} differs"
    dq, dks, dvs, dkd, dvd = [g.double().cpu().numpy() for g in g1]
    G = Hq // Hkv
    rng = np.random.default_rng(6163)
    ts = sorted(set(rng.integers(0, T, 12).tolist()) | {0, T - 1})
    groups = [(b, t, kvh) for b in range(B) for t in ts for kvh in range(Hkv)]
    rq, rkd, rvd = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), groups=groups)
    errs = {"dq": _rel_err(np.stack([dq[b, t, kvh * G:(kvh + 1) * G] for (b, t, kvh) in groups]), rq),
            "dk_depth": _rel_err(np.stack([dkd[b, t, :, kvh] for (b, t, kvh) in groups]), rkd),
            "dv_depth": _rel_err(np.stack([dvd[b, t, :, kvh] for (b, t, kvh) in groups]), rvd)}
    errs.update(key_errors("tail", np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), dks, dvs, B, Hkv,
                           tail_keys(T)))
    do = np32(dout).astype(np.float64)
    for b in range(B):
        for kvh in range(Hkv):
            sv = dvs[b, :, kvh].sum(0) + dvd[b, :, :, kvh].sum((0, 1))
            l1v = np.abs(dvs[b, :, kvh]).sum(0) + np.abs(dvd[b, :, :, kvh]).sum((0, 1))
            sk = dks[b, :, kvh].sum(0) + dkd[b, :, :, kvh].sum((0, 1))
            l1k = np.abs(dks[b, :, kvh]).sum(0) + np.abs(dkd[b, :, :, kvh]).sum((0, 1))
            errs[f"sum_dv[{b},{kvh}]"] = float((np.abs(sv - do[b, :, kvh * G:(kvh + 1) * G].sum((0, 1))) / l1v).max())
            errs[f"sum_dk[{b},{kvh}]"] = float((np.abs(sk) / l1k).max())
    tol = TOL_BWD[q.dtype]
    _say("nine pairs: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{k} error {v} > {tol}"


def test_bwd_ragged_long_grid():
    """The backward on a long grid (dQ and dK/dV tiles from the launch
    counters) with T = 20001, G = 8, L_d = 5: sampled query groups and the
    last keys (partial last key tile) against the oracle, exact sums."""
    B, T, Hq, Hkv, d, L_d = 1, 20001, 16, 2, 128, 5
    _say(f"bwd ragged long grid: B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} L_d={L_d}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype="bf16", seed=8191)
    dout = make_dout(B, T, Hq, d, dtype="bf16", seed=8192)
    dq, dks, dvs, dkd, dvd = run_fwd_bwd(q, ks, vs, kd, vd, dout)
    G = Hq // Hkv
    rng = np.random.default_rng(8193)
    ts = sorted(set(rng.integers(0, T, 16).tolist()) | {0, T - 33, T - 2, T - 1})
    groups = [(0, t, kvh) for t in ts for kvh in range(Hkv)]
    rq, rkd, rvd = moda_backward(np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), groups=groups)
    errs = {"dq": _rel_err(np.stack([dq[b, t, kvh * G:(kvh + 1) * G] for (b, t, kvh) in groups]), rq),
            "dk_depth": _rel_err(np.stack([dkd[b, t, :, kvh] for (b, t, kvh) in groups]), rkd),
            "dv_depth": _rel_err(np.stack([dvd[b, t, :, kvh] for (b, t, kvh) in groups]), rvd)}
    errs.update(key_errors("tail", np32(q), np32(ks), np32(vs), np32(kd), np32(vd), np32(dout), dks, dvs, B, Hkv,
                           tail_keys(T)))
    do = np32(dout).astype(np.float64)
    for kvh in range(Hkv):
        sv = dvs[0, :, kvh].sum(0) + dvd[0, :, :, kvh].sum((0, 1))
        l1v = np.abs(dvs[0, :, kvh]).sum(0) + np.abs(dvd[0, :, :, kvh]).sum((0, 1))
        sk = dks[0, :, kvh].sum(0) + dkd[0, :, :, kvh].sum((0, 1))
        l1k = np.abs(dks[0, :, kvh]).sum(0) + np.abs(dkd[0, :, :, kvh]).sum((0, 1))
        errs[f"sum_dv[{kvh}]"] = float((np.abs(sv - do[0, :, kvh * G:(kvh + 1) * G].sum((0, 1))) / l1v).max())
        errs[f"sum_dk[{kvh}]"] = float((np.abs(sk) / l1k).max())
    tol = TOL_BWD[q.dtype]
    _say("bwd ragged: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{k} error {v} > {tol}"
