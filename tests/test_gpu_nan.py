"""Non-finite inputs along the two masks (GPU, through the C ABI).

The causal mask lets a row at position t see the sequence keys s <= t only,
and the depth mask lets it see the depth slots of its own position only
(mhpn.cn article "动态混合深度注意力机制MoDA技术解析", section 2.2: the dual
masks keep information from leaking).  So a NaN planted in a key that a row
cannot see must leave that row bit for bit as it was, and every row that can
see it must come out NaN:

  * NaN in k_seq[b, s, kvh]: rows of kv head kvh at positions t >= s are NaN;
    rows at t < s and every row of the other kv heads are unchanged;
  * NaN in k_depth[b, t', j, kvh]: the G rows of kv head kvh at position t'
    are NaN; every other row is unchanged.

Depth slots outside a window [slot_lo, slot_hi), and the padding rows of the
packed buffers, are never read: filling them (keys and values, or the row
scales of 8-bit depth KV) with NaN must leave the forward and the backward
bit for bit unchanged.
"""
from __future__ import annotations

import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_inputs import make_dout, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def _fwd(q, ks, vs, kd, vd):
    L_d = kd.shape[2]
    kp, vp = moda.moda_pack_depth(kd, vd) if L_d else (None, None)
    out, lse = moda.moda_fwd(q, ks, vs, kp, vp, L_d)
    torch.cuda.synchronize()
    return out, lse


# dtype, B, T, Hq, Hkv, d, L_d: the bf16 matrix-core kernel (4-wave tiles) and
# the generic kernel
SHAPES = [("bf16", 2, 300, 8, 2, 128, 5), ("fp32", 1, 200, 6, 2, 64, 3), ("bf16", 1, 130, 32, 1, 128, 4)]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}_B{s[1]}_T{s[2]}_G{s[3] // s[4]}_d{s[5]}" for s in SHAPES])
def test_nan_sequence_key(shape):
    dtype, B, T, Hq, Hkv, d, L_d = shape
    G = Hq // Hkv
    q, ks, vs, kd, vd = [x.to(DEV) for x in make_inputs(B, T, Hq, Hkv, d, L_d, dtype=dtype, seed=41)]
    ref_out, ref_lse = _fwd(q, ks, vs, kd, vd)
    for (b, s, kvh) in [(B - 1, T // 2, Hkv - 1), (0, 64, 0), (0, T - 1, 0), (0, 0, Hkv - 1)]:
        _say(f"NaN k_seq[{b},{s},{kvh}] {shape}")
        ks2 = ks.clone()
        ks2[b, s, kvh, 3] = float("nan")
        out, lse = _fwd(q, ks2, vs, kd, vd)
        heads = slice(kvh * G, (kvh + 1) * G)
        seen = torch.zeros(B, T, Hq, dtype=torch.bool, device=DEV)
        seen[b, s:, heads] = True
        assert torch.isnan(out[seen]).all() and torch.isnan(lse.permute(0, 2, 1)[seen]).all()
        assert torch.equal(out[~seen], ref_out[~seen])
        assert torch.equal(lse.permute(0, 2, 1)[~seen], ref_lse.permute(0, 2, 1)[~seen])


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}_B{s[1]}_T{s[2]}_G{s[3] // s[4]}_d{s[5]}" for s in SHAPES])
def test_nan_depth_key(shape):
    dtype, B, T, Hq, Hkv, d, L_d = shape
    G = Hq // Hkv
    q, ks, vs, kd, vd = [x.to(DEV) for x in make_inputs(B, T, Hq, Hkv, d, L_d, dtype=dtype, seed=42)]
    ref_out, ref_lse = _fwd(q, ks, vs, kd, vd)
    for (b, t, j, kvh) in [(B - 1, T // 3, L_d - 1, Hkv - 1), (0, 0, 0, 0), (0, T - 1, 1, 0)]:
        _say(f"NaN k_depth[{b},{t},{j},{kvh}] {shape}")
        kd2 = kd.clone()
        kd2[b, t, j, kvh, 5] = float("nan")
        out, lse = _fwd(q, ks, vs, kd2, vd)
        seen = torch.zeros(B, T, Hq, dtype=torch.bool, device=DEV)
        seen[b, t, kvh * G:(kvh + 1) * G] = True
        assert torch.isnan(out[seen]).all() and torch.isnan(lse.permute(0, 2, 1)[seen]).all()
        assert torch.equal(out[~seen], ref_out[~seen])
        assert torch.equal(lse.permute(0, 2, 1)[~seen], ref_lse.permute(0, 2, 1)[~seen])


def _unread_rows(B, T, Hkv, L_cap, lo, hi, nkp):
    """Boolean [B, Hkv, NKp] of packed rows outside the window (or padding)."""
    n = torch.arange(nkp, device=DEV)
    slot = n % L_cap
    bad = (n >= T * L_cap) | (slot < lo) | (slot >= hi)
    return bad.view(1, 1, nkp).expand(B, Hkv, nkp)


WINDOWS = [
    # dtype, B, T, Hq, Hkv, d, L_cap, lo, hi
    ("bf16", 1, 300, 16, 2, 128, 6, 2, 5),     # matrix-core kernels, G = 8
    ("bf16", 2, 97, 6, 2, 128, 7, 0, 3),       # G = 3 (vector-unit depth-gradient kernel)
    ("fp32", 1, 150, 4, 1, 64, 5, 1, 4),       # generic kernels
    ("bf16", 1, 77, 4, 1, 128, 3, 0, 3),       # whole capacity: only the padding rows are unread
]


@pytest.mark.parametrize("case", WINDOWS, ids=[f"{c[0]}_T{c[2]}_G{c[3] // c[4]}_cap{c[6]}_{c[7]}-{c[8]}"
                                              for c in WINDOWS])
def test_unread_slots_hold_nan(case):
    dtype, B, T, Hq, Hkv, d, L_cap, lo, hi = case
    _say(f"NaN in unread slots {case}")
    q, ks, vs, kd, vd = [x.to(DEV) for x in make_inputs(B, T, Hq, Hkv, d, L_cap, dtype=dtype, seed=43)]
    dout = make_dout(B, T, Hq, d, dtype=dtype, seed=43).to(DEV)
    kp, vp = moda.moda_pack_depth(kd, vd)
    nkp = kp.numel() // (B * Hkv * d)
    bad = _unread_rows(B, T, Hkv, L_cap, lo, hi, nkp)
    kpn, vpn = kp.clone().view(B, Hkv, nkp, d), vp.clone().view(B, Hkv, nkp, d)
    kpn[bad] = float("nan")
    vpn[bad] = float("nan")
    kpn, vpn = kpn.view(-1), vpn.view(-1)
    out, lse = moda.moda_fwd_window(q, ks, vs, kp, vp, L_cap, lo, hi)
    out2, lse2 = moda.moda_fwd_window(q, ks, vs, kpn, vpn, L_cap, lo, hi)
    g = moda.moda_bwd_window(q, ks, vs, kp, vp, L_cap, lo, hi, out, lse, dout)
    g2 = moda.moda_bwd_window(q, ks, vs, kpn, vpn, L_cap, lo, hi, out, lse, dout)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for a, b_ in zip(g, g2):
        assert torch.equal(a, b_)
    # 8-bit depth KV: NaN row scales (and arbitrary codes) in the unread rows
    pq = list(moda.moda_pack_depth_q8(kd, vd))
    pn = [x.clone() for x in pq]
    for i in (0, 1):
        pn[i].view(B, Hkv, nkp, d)[bad] = 77
    for i in (2, 3):
        pn[i].view(B, Hkv, nkp)[bad] = float("nan")
    o8, l8 = moda.moda_fwd_window_q8(q, ks, vs, pq, L_cap, lo, hi)
    o8n, l8n = moda.moda_fwd_window_q8(q, ks, vs, pn, L_cap, lo, hi)
    g8 = moda.moda_bwd_window_q8(q, ks, vs, pq, L_cap, lo, hi, o8, l8, dout)
    g8n = moda.moda_bwd_window_q8(q, ks, vs, pn, L_cap, lo, hi, o8, l8, dout)
    torch.cuda.synchronize()
    assert torch.equal(o8, o8n) and torch.equal(l8, l8n)
    for a, b_ in zip(g8, g8n):
        assert torch.equal(a, b_)
