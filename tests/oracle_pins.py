"""Pins that tie the oracle to facts other than itself.

Each pin takes a forward callable with the signature of
oracle.moda_forward and returns the largest deviation it found (0.0 for exact
checks that hold).  A pin raises AssertionError when its check fails.  They are
applied to the real oracle (tests/test_oracle_pins.py) and to copies of the
oracle with planted mistakes (tests/test_oracle_mutants.py).

What each pin rests on:
  sdpa_causal      L_d = 0 reduces MoDA to ordinary causal attention (the
                   formula with only the current layer's term; mhpn.cn
                   article, section 1.2 "traditional attention"); compared
                   with torch's scaled_dot_product_attention in float64.
  sdpa_augmented   The concatenated-set softmax equals masked attention over
                   an augmented key set [sequence keys ; flattened T*L_d depth
                   keys] with the causal and same-position depth masks
                   (mhpn.cn article, section 2.2, dual masks; gist.science (de)
                   section 2, flash-compatible T x L layout).
  depth_order      A softmax over a set does not depend on the order of the
                   depth slots (section 1.2 lists them l-1 .. 0).
  prob_rows        Softmax rows are probability distributions of length
                   t + 1 + L_d.
  identical_keys   Closed form: equal keys give the mean of the values and
                   lse = z + ln n.
  brute_force      Independent scalar implementation on a grid of tiny shapes.
  merge            Unified softmax (gist.science (de) section 2, Unified
                   Softmax): inclusion-exclusion over partial key sets.
  gqa              GQA equals attention with KV heads repeated G times
                   (gist.science (de) section 2, Group-Aware Indexing).
  leak             Masks: a key at position s never reaches rows t < s; a depth
                   slot of position t' reaches only rows at t' (mhpn.cn
                   article, section 2.2, "prevents information leakage").
  saturation       A depth key aligned with the query and scaled up takes all
                   the probability mass.
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch
import torch.nn.functional as F


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _inputs(rng, B, T, Hq, Hkv, d, L_d):
    return (_rand(rng, B, T, Hq, d), _rand(rng, B, T, Hkv, d), _rand(rng, B, T, Hkv, d),
            _rand(rng, B, T, L_d, Hkv, d), _rand(rng, B, T, L_d, Hkv, d))


def _masked_lse(scores, mask):
    s = scores.masked_fill(~mask, float("-inf"))
    return torch.logsumexp(s, dim=-1)


def pin_sdpa_causal(fwd):
    rng = np.random.default_rng(11)
    worst = 0.0
    for (B, T, Hq, Hkv, d) in [(2, 7, 4, 2, 8), (1, 9, 3, 1, 5), (1, 1, 2, 2, 4)]:
        q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, 0)
        out, lse = fwd(q, ks, vs, kd, vd)
        G = Hq // Hkv
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(ks).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
        tv = torch.from_numpy(vs).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
        ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
        ref = ref.permute(0, 2, 1, 3).numpy()
        scores = (tq @ tk.transpose(-1, -2)) / math.sqrt(d)
        causal = torch.ones(T, T, dtype=torch.bool).tril()
        ref_lse = _masked_lse(scores, causal).numpy()
        e_out = float(np.abs(out - ref).max())
        e_lse = float(np.abs(lse - ref_lse).max())
        # first position: its only key is itself, so out = v_seq[:, 0]
        e_t0 = float(np.abs(out[:, 0] - np.repeat(vs[:, 0], G, axis=1)).max())
        assert e_out <= 1e-12, f"out vs causal SDPA: {e_out}"
        assert e_lse <= 1e-12, f"lse vs masked logsumexp: {e_lse}"
        assert e_t0 <= 1e-14, f"t=0 row: {e_t0}"
        worst = max(worst, e_out, e_lse, e_t0)
    return worst


def pin_sdpa_augmented(fwd):
    rng = np.random.default_rng(12)
    worst = 0.0
    for (B, T, Hq, Hkv, d, L_d) in [(2, 6, 4, 2, 8, 3), (1, 5, 3, 3, 4, 1), (1, 4, 8, 1, 6, 5)]:
        q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
        out, lse = fwd(q, ks, vs, kd, vd)
        G = Hq // Hkv
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        # augmented key axis: T sequence keys, then T*L_d depth keys (t-major)
        kdf = torch.from_numpy(kd).permute(0, 3, 1, 2, 4).reshape(B, Hkv, T * L_d, d)
        vdf = torch.from_numpy(vd).permute(0, 3, 1, 2, 4).reshape(B, Hkv, T * L_d, d)
        tk = torch.cat([torch.from_numpy(ks).permute(0, 2, 1, 3), kdf], dim=2).repeat_interleave(G, dim=1)
        tv = torch.cat([torch.from_numpy(vs).permute(0, 2, 1, 3), vdf], dim=2).repeat_interleave(G, dim=1)
        mask = torch.zeros(T, T + T * L_d, dtype=torch.bool)
        for t in range(T):
            mask[t, : t + 1] = True
            mask[t, T + t * L_d: T + (t + 1) * L_d] = True
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask).permute(0, 2, 1, 3).numpy()
        ref_lse = _masked_lse((tq @ tk.transpose(-1, -2)) / math.sqrt(d), mask).numpy()
        e_out = float(np.abs(out - ref).max())
        e_lse = float(np.abs(lse - ref_lse).max())
        assert e_out <= 1e-12, f"out vs augmented SDPA: {e_out}"
        assert e_lse <= 1e-12, f"lse vs augmented logsumexp: {e_lse}"
        worst = max(worst, e_out, e_lse)
    return worst


def pin_depth_order(fwd):
    rng = np.random.default_rng(13)
    q, ks, vs, kd, vd = _inputs(rng, 2, 6, 4, 2, 8, 5)
    out, lse = fwd(q, ks, vs, kd, vd)
    perm = rng.permutation(5)
    out2, lse2 = fwd(q, ks, vs, kd[:, :, perm], vd[:, :, perm])
    e = max(float(np.abs(out - out2).max()), float(np.abs(lse - lse2).max()))
    assert e <= 1e-13, f"depth order changed the result: {e}"
    # a permutation of only the keys (values fixed) must change it
    out3, _ = fwd(q, ks, vs, kd[:, :, perm], vd)
    assert float(np.abs(out - out3).max()) > 1e-6, "key/value pairing not respected"
    return e


def pin_prob_rows(fwd):
    rng = np.random.default_rng(14)
    B, T, Hq, Hkv, d, L_d = 1, 6, 4, 2, 8, 3
    q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
    rows = [(0, t, h) for t in range(T) for h in range(Hq)]
    _, _, probs = fwd(q, ks, vs, kd, vd, rows=rows, return_probs=True)
    worst = 0.0
    for (b, t, h), p in zip(rows, probs):
        p = np.asarray(p)
        assert p.shape == (t + 1 + L_d,), f"row {(b, t, h)} has {p.shape} probabilities"
        assert float(p.min()) >= 0.0
        worst = max(worst, abs(float(p.sum()) - 1.0))
    assert worst <= 1e-13, f"probabilities do not sum to 1: {worst}"
    return worst


def pin_identical_keys(fwd):
    rng = np.random.default_rng(15)
    B, T, Hq, Hkv, d, L_d = 1, 6, 4, 2, 8, 3
    worst = 0.0
    for (t, h, zero_q) in [(0, 0, False), (3, 1, False), (5, 3, True), (4, 2, False)]:
        q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
        kvh = h // (Hq // Hkv)
        c = rng.standard_normal(d)
        ks[0, : t + 1, kvh] = c
        kd[0, t, :, kvh] = c
        if zero_q:
            q[0, t, h] = 0.0
        out, lse = fwd(q, ks, vs, kd, vd, rows=[(0, t, h)])
        n = t + 1 + L_d
        mean_v = (vs[0, : t + 1, kvh].sum(axis=0) + vd[0, t, :, kvh].sum(axis=0)) / n
        z = float(np.dot(q[0, t, h], c)) / math.sqrt(d)
        e_out = float(np.abs(out[0] - mean_v).max())
        e_lse = abs(float(lse[0]) - (z + math.log(n)))
        assert e_out <= 1e-13, f"identical keys: out not the mean ({e_out})"
        assert e_lse <= 1e-13, f"identical keys: lse != z + ln n ({e_lse})"
        worst = max(worst, e_out, e_lse)
    return worst


def pin_brute_force(fwd, scalar):
    rng = np.random.default_rng(16)
    worst = 0.0
    grid = itertools.product([1, 2], [1, 4, 9], [(2, 1), (4, 2), (3, 3)], [3, 8], [0, 1, 4])
    for (B, T, (Hq, Hkv), d, L_d) in grid:
        q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
        out, lse = fwd(q, ks, vs, kd, vd)
        so, sl = scalar(q, ks, vs, kd, vd)
        e = max(float(np.abs(out - np.array(so)).max()), float(np.abs(lse - np.array(sl)).max()))
        assert e <= 1e-12, f"brute force {(B, T, Hq, Hkv, d, L_d)}: {e}"
        worst = max(worst, e)
    return worst


def pin_merge(fwd):
    """Unified softmax by inclusion-exclusion over the key set.

    With S = sequence keys and depth slots split into A and B, the
    unnormalised sums add up:  e^lse(S+A+B) = e^lse(S+A) + e^lse(S+B) - e^lse(S)
    and likewise for e^lse * out.  Separate normalisation of the two sets, or
    any weighting between them, breaks this.
    """
    rng = np.random.default_rng(17)
    B, T, Hq, Hkv, d, L_d = 2, 5, 4, 2, 8, 4
    q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
    o_all, l_all = fwd(q, ks, vs, kd, vd)
    o_s, l_s = fwd(q, ks, vs, kd[:, :, :0], vd[:, :, :0])
    o_a, l_a = fwd(q, ks, vs, kd[:, :, :1], vd[:, :, :1])
    o_b, l_b = fwd(q, ks, vs, kd[:, :, 1:], vd[:, :, 1:])
    # lse is [B,Hq,T]; bring to [B,T,Hq,1] to weight out
    w = lambda l: np.exp(np.transpose(l, (0, 2, 1)))[..., None]  # noqa: E731
    z_all = np.exp(l_all)
    z_mix = np.exp(l_a) + np.exp(l_b) - np.exp(l_s)
    e_z = float(np.abs(z_all - z_mix).max() / np.abs(z_all).max())
    num = w(l_a) * o_a + w(l_b) * o_b - w(l_s) * o_s
    e_o = float(np.abs(num / w(l_all) - o_all).max())
    assert e_z <= 1e-10, f"merge identity on the normaliser: {e_z}"
    assert e_o <= 1e-9, f"merge identity on the output: {e_o}"
    return max(e_z, e_o)


def pin_gqa(fwd):
    rng = np.random.default_rng(18)
    B, T, Hq, Hkv, d, L_d = 1, 6, 6, 2, 8, 2
    G = Hq // Hkv
    q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
    out, lse = fwd(q, ks, vs, kd, vd)
    out_x, lse_x = fwd(q, np.repeat(ks, G, axis=2), np.repeat(vs, G, axis=2),
                       np.repeat(kd, G, axis=3), np.repeat(vd, G, axis=3))
    e = max(float(np.abs(out - out_x).max()), float(np.abs(lse - lse_x).max()))
    assert e <= 1e-13, f"GQA vs repeated KV: {e}"
    # equal queries inside one group give equal rows
    q2 = q.copy()
    q2[:, :, 1] = q2[:, :, 0]
    out2, lse2 = fwd(q2, ks, vs, kd, vd)
    assert np.array_equal(out2[:, :, 0], out2[:, :, 1]) and np.array_equal(lse2[:, 0], lse2[:, 1])
    return e


def pin_leak(fwd):
    rng = np.random.default_rng(19)
    B, T, Hq, Hkv, d, L_d = 2, 7, 4, 2, 8, 3
    q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
    out, lse = fwd(q, ks, vs, kd, vd)
    s = 4
    ks2, vs2 = ks.copy(), vs.copy()
    ks2[1, s] += 3.0
    vs2[1, s] -= 2.0
    out2, lse2 = fwd(q, ks2, vs2, kd, vd)
    assert np.array_equal(out2[1, :s], out[1, :s]) and np.array_equal(lse2[1, :, :s], lse[1, :, :s]), \
        "a future sequence key reached an earlier row"
    assert np.array_equal(out2[0], out[0]), "a sequence key crossed batches"
    assert np.all(np.abs(out2[1, s:] - out[1, s:]).max(axis=-1) > 0.0), "key at s did not reach rows t >= s"
    tp = 2
    kd2, vd2 = kd.copy(), vd.copy()
    kd2[0, tp] += 3.0
    vd2[0, tp] -= 2.0
    out3, lse3 = fwd(q, ks, vs, kd2, vd2)
    others = [t for t in range(T) if t != tp]
    assert np.array_equal(out3[0, others], out[0, others]) and np.array_equal(lse3[0][:, others], lse[0][:, others]), \
        "a depth slot reached another position"
    assert np.array_equal(out3[1], out[1]), "a depth slot crossed batches"
    assert np.all(np.abs(out3[0, tp] - out[0, tp]).max(axis=-1) > 0.0), "depth slot did not reach its own position"
    return 0.0


def pin_saturation(fwd):
    rng = np.random.default_rng(20)
    B, T, Hq, Hkv, d, L_d = 1, 5, 2, 2, 8, 3
    q, ks, vs, kd, vd = _inputs(rng, B, T, Hq, Hkv, d, L_d)
    t, h, j = 3, 1, 2
    errs = []
    for alpha in [1.0, 4.0, 16.0, 64.0, 256.0]:
        kd2 = kd.copy()
        kd2[0, t, j, h] = alpha * q[0, t, h]
        out, _ = fwd(q, ks, vs, kd2, vd, rows=[(0, t, h)])
        errs.append(float(np.abs(out[0] - vd[0, t, j, h]).max()))
    assert all(b <= a + 1e-15 for a, b in zip(errs, errs[1:])), f"not monotone: {errs}"
    assert errs[-1] <= 1e-9, f"no saturation: {errs}"
    return errs[-1]


PINS = {
    "sdpa_causal": pin_sdpa_causal,
    "sdpa_augmented": pin_sdpa_augmented,
    "depth_order": pin_depth_order,
    "prob_rows": pin_prob_rows,
    "identical_keys": pin_identical_keys,
    "merge": pin_merge,
    "gqa": pin_gqa,
    "leak": pin_leak,
    "saturation": pin_saturation,
}
