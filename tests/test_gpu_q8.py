"""GPU parity of 8-bit depth KV: moda_pack_depth_q8 codes and scales bit for
bit against the oracle's quantisation, moda_fwd_q8 against the forward oracle
on the dequantised depth KV, and moda_bwd_q8 against the backward oracle on
the same dequantised depth KV."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_check import TOL, key_errors, np32, tail_keys
from moda_inputs import make_dout, make_inputs, sample_rows, workload
from oracle import moda_backward, moda_forward
from oracle.moda_quant import dequantize_rows, quantize_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _packed_rows(x):
    """Logical [B,T,L,Hkv,d] -> packed row order [B,Hkv,T*L,d] (no padding)."""
    B, T, L, Hkv, d = x.shape
    return np.transpose(x, (0, 3, 1, 2, 4)).reshape(B, Hkv, T * L, d)


def _ref_q8(kd, vd):
    """Oracle codes / scales in the packed order, with zero padding rows."""
    B, T, L, Hkv, d = kd.shape
    NKp = (T * L + 31) // 32 * 32
    out = []
    for x in (kd, vd):
        codes, scales = quantize_rows(_packed_rows(np32(x)))
        c = np.zeros((B, Hkv, NKp, d), np.int8)
        s = np.zeros((B, Hkv, NKp), np.float32)
        c[:, :, :T * L] = codes
        s[:, :, :T * L] = scales
        out += [c.reshape(-1), s.reshape(-1)]
    return out


def _with_zero_rows(kd, vd):
    kd = kd.clone()
    vd = vd.clone()
    kd[0, 0, 0] = 0          # all-zero key rows (scale 0)
    vd[0, -1, -1] = 0
    return kd, vd


@pytest.mark.parametrize("case", [("bf16", 2, 37, 3, 128, 5), ("fp32", 1, 64, 2, 64, 3),
                                  ("bf16", 1, 40, 1, 64, 24), ("fp32", 1, 9, 2, 128, 2)])
def test_pack_q8_bitwise(case):
    dtype, B, T, Hkv, d, L = case
    _say(f"pack q8 {case}")
    _, _, _, kd, vd = make_inputs(B, T, Hkv, Hkv, d, L, dtype=dtype, seed=9)
    kd, vd = _with_zero_rows(kd, vd)
    kq, vq, ks, vs = moda.moda_pack_depth_q8(kd.cuda(), vd.cuda())
    torch.cuda.synchronize()
    rkq, rks, rvq, rvs = _ref_q8(kd, vd)
    assert np.array_equal(kq.cpu().numpy(), rkq)
    assert np.array_equal(vq.cpu().numpy(), rvq)
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    assert np.array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32))
    # the same codes written into caller buffers that held other bytes
    out = tuple(torch.full_like(t, 7) for t in (kq, vq, ks, vs))
    got = moda.moda_pack_depth_q8(kd.cuda(), vd.cuda(), out=out)
    torch.cuda.synchronize()
    assert all(g is o for g, o in zip(got, out))
    for a, b in zip(out, (kq, vq, ks, vs)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_pack_q8_ties_and_near_ties(dtype):
    """Rows whose quotients x / scale land exactly on half-integers (scale 1:
    row maximum 127) and rows with quotients a few ulps either side of
    half-integers: codes bit for bit the oracle's (ties to even), which takes
    the kernel's exact-division path."""
    _say(f"q8 ties {dtype}")
    B, T, L, Hkv, d = 1, 40, 3, 2, 128
    g = torch.Generator().manual_seed(17)
    x = torch.randn(B, T, L, Hkv, d, generator=g, dtype=torch.float32)
    halves = torch.arange(-64, 64, dtype=torch.float32) + 0.5            # -63.5 .. 63.5
    x[0, :10, :, :, :] = halves                                           # exact ties after max = 127
    x[0, :10, :, :, 0] = 127.0
    # quotients just off the half-integers: scale = 127 / 127 * s for s = 1 + 2^-k
    for k, t in zip(range(6, 16), range(10, 20)):
        sc = 1.0 + 2.0 ** -k
        x[0, t, :, :, :] = (halves + 2.0 ** -k) * sc
        x[0, t, :, :, 0] = 127.0 * sc
    if dtype == "bf16":
        x = x.to(torch.bfloat16)
    kd, vd = x, x.flip(-1).contiguous()
    kq, vq, ks, vs = moda.moda_pack_depth_q8(kd.cuda(), vd.cuda())
    torch.cuda.synchronize()
    rkq, rks, rvq, rvs = _ref_q8(kd, vd)
    assert np.array_equal(kq.cpu().numpy(), rkq)
    assert np.array_equal(vq.cpu().numpy(), rvq)
    assert np.array_equal(ks.cpu().numpy().view(np.uint32), rks.view(np.uint32))
    assert np.array_equal(vs.cpu().numpy().view(np.uint32), rvs.view(np.uint32))


def _deq_logical(kd):
    """Oracle dequantised depth tensor in the logical layout (float64)."""
    codes, scales = quantize_rows(np32(kd))
    return dequantize_rows(codes, scales)


def _run(q, ks, vs, kd, vd):
    dev = torch.device("cuda:0")
    L = kd.shape[2]
    packed = moda.moda_pack_depth_q8(kd.to(dev), vd.to(dev)) if L > 0 else None
    out, lse = moda.moda_fwd_q8(q.to(dev), ks.to(dev), vs.to(dev), packed, L)
    torch.cuda.synchronize()
    return out, lse


def _check(name, dtype, out, lse, ref_out, ref_lse):
    tol = TOL[dtype]
    eo = float(np.abs(out.double().cpu().numpy() - ref_out).max())
    el = float(np.abs(lse.double().cpu().numpy() - ref_lse).max())
    _say(f"{name}: max|out-ref| = {eo:.3e}  max|lse-ref| = {el:.3e}  (tol {tol:g})")
    assert eo <= tol and el <= tol


CASES = [
    ("fp32_T128_G4_d64_L3", "fp32", 1, 128, 4, 1, 64, 3),
    ("bf16_T300_G4_d128_L5", "bf16", 1, 300, 8, 2, 128, 5),
    ("bf16_B2_T97_G3_d128_L4", "bf16", 2, 97, 6, 2, 128, 4),
    ("bf16_T130_G32_d64_L6", "bf16", 1, 130, 32, 1, 64, 6),
    ("fp32_T77_G2_d128_L7", "fp32", 1, 77, 4, 2, 128, 7),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_fwd_q8_parity(case):
    name, dtype, B, T, Hq, Hkv, d, L = case
    _say(f"fwd q8 {name}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L, dtype=dtype, seed=70 + T)
    kd, vd = _with_zero_rows(kd, vd)
    out, lse = _run(q, ks, vs, kd, vd)
    ref_out, ref_lse = moda_forward(np32(q), np32(ks), np32(vs), _deq_logical(kd), _deq_logical(vd))
    _check(name, q.dtype, out, lse, ref_out, ref_lse)


def test_fwd_q8_without_depth_is_fwd():
    q, ks, vs, kd, vd = make_inputs(1, 100, 4, 2, 128, 0, dtype="bf16", seed=3)
    _say("fwd q8 with L_d = 0")
    o1, l1 = _run(q, ks, vs, kd, vd)
    o2, l2 = moda.moda_fwd(q.cuda(), ks.cuda(), vs.cuda(), None, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["bf16_B1_T4096_Hq16_Hkv2_d128_L24", "bf16_B1_T65536_Hq16_Hkv2_d128_L24"])
def test_fwd_q8_workload(name):
    w = workload(name)
    _say(f"fwd q8 workload {name}")
    q, ks, vs, kd, vd = make_inputs(w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"], dtype=w["dtype"],
                                    seed=w["seed"])
    out, lse = _run(q, ks, vs, kd, vd)
    if w["T"] <= 4096:
        rows = None
    else:
        rows = sample_rows(w["B"], w["T"], w["Hq"], n=1024, seed=w["seed"] + 17)
    dk, dv = _deq_logical(kd), _deq_logical(vd)
    if rows is None:
        ref_out, ref_lse = moda_forward(np32(q), np32(ks), np32(vs), dk, dv)
        _check(name, q.dtype, out, lse, ref_out, ref_lse)
    else:
        ref_out, ref_lse = moda_forward(np32(q), np32(ks), np32(vs), dk, dv, rows=rows)
        r = np.asarray(rows)
        o = out[torch.from_numpy(r[:, 0]).cuda(), torch.from_numpy(r[:, 1]).cuda(), torch.from_numpy(r[:, 2]).cuda()]
        l = lse[torch.from_numpy(r[:, 0]).cuda(), torch.from_numpy(r[:, 2]).cuda(), torch.from_numpy(r[:, 1]).cuda()]
        _check(name + " (sampled)", q.dtype, o, l, ref_out, ref_lse)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64), ("bf16", 64)])
def test_fwd_q8_bitwise_on_exact_codes(dtype, d):
    """Depth values that are integer multiples (|k| <= 127, row max 127) of a
    power of two quantise exactly, so the 8-bit forward must give bit for bit
    the output of the plain forward on the same values."""
    _say(f"fwd q8 exact codes {dtype} d={d}")
    B, T, Hq, Hkv, L = 1, 150, 8, 2, 5
    q, ks, vs, _, _ = make_inputs(B, T, Hq, Hkv, d, 0, dtype=dtype, seed=11)
    g = torch.Generator().manual_seed(12)
    td = q.dtype
    codes = torch.randint(-127, 128, (2, B, T, L, Hkv, d), generator=g)
    codes[..., 0] = 127
    kd = (codes[0].float() * 2.0 ** -6).to(td)
    vd = (codes[1].float() * 2.0 ** -5).to(td)
    dev = torch.device("cuda:0")
    o1, l1 = _run(q, ks, vs, kd, vd)
    kp, vp = moda.moda_pack_depth(kd.to(dev), vd.to(dev))
    o2, l2 = moda.moda_fwd(q.to(dev), ks.to(dev), vs.to(dev), kp, vp, L)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_append_q8_equals_pack_q8():
    """Appending slots 0..L-1 one layer at a time into zero-filled 8-bit
    buffers gives bit for bit the buffers of moda_pack_depth_q8."""
    B, T, Hkv, d, L = 2, 45, 2, 128, 5
    _say("append q8 vs pack q8")
    _, _, _, kd, vd = make_inputs(B, T, Hkv, Hkv, d, L, dtype="bf16", seed=21)
    kd, vd = _with_zero_rows(kd, vd)
    ref = moda.moda_pack_depth_q8(kd.cuda(), vd.cuda())
    n = moda.depth_packed_elems(B, T, Hkv, d, L)
    buf = (torch.zeros(n, dtype=torch.int8, device="cuda"), torch.zeros(n, dtype=torch.int8, device="cuda"),
           torch.zeros(n // d, dtype=torch.float32, device="cuda"), torch.zeros(n // d, dtype=torch.float32, device="cuda"))
    for j in range(L):
        moda.moda_append_depth_q8(kd[:, :, j].contiguous().cuda(), vd[:, :, j].contiguous().cuda(), buf, L, j)
    torch.cuda.synchronize()
    for a, b in zip(buf, ref):
        assert torch.equal(a.view(torch.int8) if a.dtype == torch.int8 else a.view(torch.int32),
                           b.view(torch.int8) if b.dtype == torch.int8 else b.view(torch.int32))


@pytest.mark.parametrize("case", [("bf16", 1, 200, 8, 2, 128, 6, 2, 5), ("fp32", 1, 90, 4, 1, 64, 4, 0, 4),
                                  ("bf16", 2, 70, 4, 2, 64, 8, 7, 8)])
def test_fwd_window_q8_parity(case):
    dtype, B, T, Hq, Hkv, d, L_cap, lo, hi = case
    _say(f"fwd window q8 {case}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_cap, dtype=dtype, seed=90 + T)
    dev = torch.device("cuda:0")
    packed = moda.moda_pack_depth_q8(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd_window_q8(q.to(dev), ks.to(dev), vs.to(dev), packed, L_cap, lo, hi)
    torch.cuda.synchronize()
    ref_out, ref_lse = moda_forward(np32(q), np32(ks), np32(vs), _deq_logical(kd)[:, :, lo:hi],
                                    _deq_logical(vd)[:, :, lo:hi])
    _check(f"window q8 {case}", q.dtype, out, lse, ref_out, ref_lse)


# max |gpu - oracle| / max(1, max |oracle|) per gradient (as for moda_bwd)
TOL_BWD = {torch.float32: 1e-5, torch.bfloat16: 1.5e-2}
BWD_CASES = [
    # dtype, B, T, Hq, Hkv, d, L_cap, slot_lo, slot_hi
    ("bf16", 1, 200, 16, 2, 128, 5, 0, 5),    # matrix-core depth kernel (G = 8)
    ("bf16", 2, 97, 6, 2, 128, 4, 0, 4),      # G = 3: vector-unit depth kernel
    ("fp32", 1, 90, 4, 1, 64, 3, 0, 3),       # generic kernels throughout
    ("bf16", 1, 150, 8, 2, 128, 6, 2, 5),     # a window of the slots
    ("fp32", 1, 70, 6, 2, 128, 5, 1, 4),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[
    f"{c[0]}_B{c[1]}_T{c[2]}_Hq{c[3]}_Hkv{c[4]}_d{c[5]}_cap{c[6]}_{c[7]}-{c[8]}" for c in BWD_CASES])
def test_bwd_q8_parity(case):
    dtype, B, T, Hq, Hkv, d, L_cap, lo, hi = case
    _say(f"bwd q8 {case}")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_cap, dtype=dtype, seed=110 + T)
    kd, vd = _with_zero_rows(kd, vd)
    dout = make_dout(B, T, Hq, d, dtype=dtype, seed=110 + T)
    dev = torch.device("cuda:0")
    qd, ksd, vsd, dd = q.to(dev), ks.to(dev), vs.to(dev), dout.to(dev)
    packed = moda.moda_pack_depth_q8(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd_window_q8(qd, ksd, vsd, packed, L_cap, lo, hi)
    grads = moda.moda_bwd_window_q8(qd, ksd, vsd, packed, L_cap, lo, hi, out, lse, dd)
    torch.cuda.synchronize()
    refs = moda_backward(np32(q), np32(ks), np32(vs), _deq_logical(kd)[:, :, lo:hi],
                         _deq_logical(vd)[:, :, lo:hi], np32(dout))
    tol = TOL_BWD[q.dtype]
    for nm, g, r in zip(("dq", "dk_seq", "dv_seq", "dk_depth", "dv_depth"), grads, refs):
        e = float(np.abs(g.double().cpu().numpy() - r).max()) / max(1.0, float(np.abs(r).max()))
        _say(f"  {nm}: {e:.2e}  (tol {tol:g})")
        assert e <= tol, f"{case}: {nm} error {e} > {tol}"


def test_bwd_q8_full_window_is_bwd_q8():
    # moda_bwd_q8(..., L_d) is moda_bwd_window_q8(..., L_cap = L_d, 0, L_d): same bits
    q, ks, vs, kd, vd = make_inputs(1, 120, 8, 2, 128, 4, dtype="bf16", seed=5)
    dout = make_dout(1, 120, 8, 128, dtype="bf16", seed=5)
    dev = torch.device("cuda:0")
    qd, ksd, vsd, dd = q.to(dev), ks.to(dev), vs.to(dev), dout.to(dev)
    packed = moda.moda_pack_depth_q8(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd_q8(qd, ksd, vsd, packed, 4)
    a = moda.moda_bwd_q8(qd, ksd, vsd, packed, 4, out, lse, dd)
    b = moda.moda_bwd_window_q8(qd, ksd, vsd, packed, 4, 0, 4, out, lse, dd)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_bwd_q8_workload_sampled():
    """B = 2, T = 16K workload over 8-bit depth KV: the query and depth-slot
    gradients of sampled (b, t, kv head) groups against the oracle's
    per-group form on the dequantised depth KV, the sequence-key gradients of
    the last keys against its per-key form, and the exact gradient sums
    (sum of dv over all keys = sum of dout, sum of dk = 0) per (b, kv head)."""
    w = workload("bf16_B2_T16384_Hq16_Hkv2_d128_L24")
    _say(f"bwd q8 {w['name']} (sampled groups + gradient sums)")
    B, T, Hq, Hkv, d, L = w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"]
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L, dtype=w["dtype"], seed=w["seed"])
    dout = make_dout(B, T, Hq, d, dtype=w["dtype"], seed=w["seed"])
    dev = torch.device("cuda:0")
    qd, ksd, vsd, dd = q.to(dev), ks.to(dev), vs.to(dev), dout.to(dev)
    packed = moda.moda_pack_depth_q8(kd.to(dev), vd.to(dev))
    out, lse = moda.moda_fwd_q8(qd, ksd, vsd, packed, L)
    dq, dks, dvs, dkd, dvd = moda.moda_bwd_q8(qd, ksd, vsd, packed, L, out, lse, dd)
    torch.cuda.synchronize()
    G = Hq // Hkv
    rng = np.random.default_rng(w["seed"] + 13)
    ts = sorted(set(rng.integers(0, T, 20).tolist()) | {0, 1, 63, T - 1})
    groups = [(int(rng.integers(0, B)), t, kvh) for t in ts for kvh in range(Hkv)]
    kdq, vdq = _deq_logical(kd), _deq_logical(vd)
    rq, rkd, rvd = moda_backward(np32(q), np32(ks), np32(vs), kdq, vdq, np32(dout), groups=groups)
    gq = np.stack([dq[b, t, kvh * G:(kvh + 1) * G].double().cpu().numpy() for (b, t, kvh) in groups])
    gkd = np.stack([dkd[b, t, :, kvh].double().cpu().numpy() for (b, t, kvh) in groups])
    gvd = np.stack([dvd[b, t, :, kvh].double().cpu().numpy() for (b, t, kvh) in groups])
    tol = TOL_BWD[q.dtype]

    def rel(a, r):
        return float(np.abs(a - r).max()) / max(1.0, float(np.abs(r).max()))

    errs = {"dq": rel(gq, rq), "dk_depth": rel(gkd, rkd), "dv_depth": rel(gvd, rvd)}
    # sequence-key gradients element by element at the last keys (both batches)
    errs.update(key_errors("tail", np32(q), np32(ks), np32(vs), kdq, vdq, np32(dout), dks, dvs, B, Hkv,
                           tail_keys(T)))
    do = np32(dout).astype(np.float64)
    dvs_, dks_ = dvs.double().cpu().numpy(), dks.double().cpu().numpy()
    dvd_, dkd_ = dvd.double().cpu().numpy(), dkd.double().cpu().numpy()
    for b in range(B):
        for kvh in range(Hkv):
            sv = dvs_[b, :, kvh].sum(0) + dvd_[b, :, :, kvh].sum((0, 1))
            ref = do[b, :, kvh * G:(kvh + 1) * G].sum((0, 1))
            l1v = np.abs(dvs_[b, :, kvh]).sum(0) + np.abs(dvd_[b, :, :, kvh]).sum((0, 1))
            sk = dks_[b, :, kvh].sum(0) + dkd_[b, :, :, kvh].sum((0, 1))
            l1k = np.abs(dks_[b, :, kvh]).sum(0) + np.abs(dkd_[b, :, :, kvh]).sum((0, 1))
            errs[f"sum_dv[{b},{kvh}]"] = float((np.abs(sv - ref) / l1v).max())
            errs[f"sum_dk[{b},{kvh}]"] = float((np.abs(sk) / l1k).max())
    _say(f"{w['name']} q8: " + "  ".join(f"{k} {v:.2e}" for k, v in errs.items()) + f"  (tol {tol:g})")
    for k, v in errs.items():
        assert v <= tol, f"{k} error {v} > {tol}"
