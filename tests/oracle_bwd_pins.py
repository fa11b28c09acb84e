"""Pins that tie the backward oracle to facts other than itself.

Each pin takes a backward callable with the signature of
oracle.moda_backward and raises AssertionError when its check fails.  They
are applied to the real oracle (tests/test_oracle_backward.py) and to copies
with planted mistakes (same file).

What each pin rests on:
  finite_diff     Central differences of the forward oracle (itself pinned by
                  tests/oracle_pins.py): the gradient of L = <out, dout> along
                  random directions, and element by element on a tiny shape.
  autograd        torch autograd of float64 attention over the augmented key
                  set [sequence keys ; flattened T*L_d depth keys] with the
                  causal and same-position masks (a library routine), with
                  and without depth, GQA by repeating KV heads.
  sums            Exact identities of the softmax: every row's weights sum to
                  one, so the value gradients of one kv head sum to the sum of
                  dout over its rows; the score gradients of a row sum to zero,
                  so the key gradients of one kv head sum to zero.
  groups          The per-group form (query rows and depth slots of one
                  (b, t, kv head)) equals the same entries of the full form.
  keys            The per-key form (sequence-key gradients summed column by
                  column over the rows that see the key, through lse and
                  Delta = dout . out) equals the same entries of the full form,
                  which the pins above tie to finite differences and autograd.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import moda_forward


def _inputs(rng, B, T, Hq, Hkv, d, L_d):
    r = rng.standard_normal
    return (r((B, T, Hq, d)), r((B, T, Hkv, d)), r((B, T, Hkv, d)),
            r((B, T, L_d, Hkv, d)), r((B, T, L_d, Hkv, d)), r((B, T, Hq, d)))


def _loss(x, dout):
    out, _ = moda_forward(*x)
    return float((out * dout).sum())


def pin_finite_diff(bwd):
    rng = np.random.default_rng(21)
    worst = 0.0
    # random directions on a few shapes
    for (B, T, Hq, Hkv, d, L_d) in [(1, 5, 4, 2, 6, 3), (2, 4, 3, 1, 5, 2), (1, 6, 2, 2, 4, 0)]:
        *x, dout = _inputs(rng, B, T, Hq, Hkv, d, L_d)
        grads = bwd(*x, dout)
        h = 1e-5
        for i in range(5):
            for _ in range(2):
                u = rng.standard_normal(x[i].shape)
                xp = [a.copy() for a in x]
                xm = [a.copy() for a in x]
                xp[i] += h * u
                xm[i] -= h * u
                fd = (_loss(xp, dout) - _loss(xm, dout)) / (2 * h)
                an = float((grads[i] * u).sum())
                err = abs(fd - an) / max(1.0, abs(fd))
                worst = max(worst, err)
                assert err <= 1e-7, f"input {i}: directional derivative {an} vs finite difference {fd}"
    # element by element on a tiny shape
    *x, dout = _inputs(rng, 1, 3, 2, 1, 3, 2)
    grads = bwd(*x, dout)
    h = 1e-6
    for i in range(5):
        num = np.zeros_like(x[i])
        for idx in np.ndindex(x[i].shape):
            xp = [a.copy() for a in x]
            xm = [a.copy() for a in x]
            xp[i][idx] += h
            xm[i][idx] -= h
            num[idx] = (_loss(xp, dout) - _loss(xm, dout)) / (2 * h)
        err = float(np.abs(num - grads[i]).max())
        worst = max(worst, err)
        assert err <= 1e-7, f"input {i}: element-wise gradient error {err}"
    return worst


def _torch_grads(q, ks, vs, kd, vd, dout):
    """Autograd of float64 masked attention over the augmented key set."""
    B, T, Hq, d = q.shape
    Hkv = ks.shape[2]
    L_d = kd.shape[2]
    G = Hq // Hkv
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, ks, vs, kd, vd)]
    tq, tks, tvs, tkd, tvd = t
    # augmented keys per kv head: T sequence keys, then T*L_d depth keys (t-major)
    kaug = torch.cat([tks, tkd.reshape(B, T * L_d, Hkv, d)], dim=1)   # [B, T+T*L_d, Hkv, d]
    vaug = torch.cat([tvs, tvd.reshape(B, T * L_d, Hkv, d)], dim=1)
    kaug = kaug.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)       # [B, Hq, N, d]
    vaug = vaug.permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    qq = tq.permute(0, 2, 1, 3)                                       # [B, Hq, T, d]
    pos = torch.arange(T)
    seq_ok = pos[None, :] <= pos[:, None]                             # [T, T]
    dpos = torch.arange(T * L_d) // max(L_d, 1)
    dep_ok = dpos[None, :] == pos[:, None]                            # [T, T*L_d]
    mask = torch.cat([seq_ok, dep_ok], dim=1)
    out = torch.nn.functional.scaled_dot_product_attention(qq, kaug, vaug, attn_mask=mask)
    out = out.permute(0, 2, 1, 3)
    out.backward(torch.tensor(dout, dtype=torch.float64))
    return [a.grad.numpy() for a in t]


def pin_autograd(bwd):
    rng = np.random.default_rng(22)
    worst = 0.0
    for shape in [(2, 7, 4, 2, 8, 3), (1, 9, 6, 3, 5, 1), (1, 6, 4, 1, 4, 0), (1, 1, 2, 2, 4, 2)]:
        *x, dout = _inputs(rng, *shape)
        got = bwd(*x, dout)
        ref = _torch_grads(*x, dout)
        for i in range(5):
            err = float(np.abs(got[i] - ref[i]).max()) if got[i].size else 0.0
            worst = max(worst, err)
            assert err <= 1e-12, f"shape {shape}, gradient {i}: {err} vs torch autograd"
    return worst


def pin_sums(bwd):
    rng = np.random.default_rng(23)
    worst = 0.0
    for (B, T, Hq, Hkv, d, L_d) in [(2, 8, 4, 2, 6, 3), (1, 11, 3, 1, 4, 5)]:
        *x, dout = _inputs(rng, B, T, Hq, Hkv, d, L_d)
        dq, dks, dvs, dkd, dvd = bwd(*x, dout)
        G = Hq // Hkv
        for b in range(B):
            for kvh in range(Hkv):
                sv = dvs[b, :, kvh].sum(0) + dvd[b, :, :, kvh].sum((0, 1))
                ref = dout[b, :, kvh * G:(kvh + 1) * G].sum((0, 1))
                sk = dks[b, :, kvh].sum(0) + dkd[b, :, :, kvh].sum((0, 1))
                e = max(float(np.abs(sv - ref).max()), float(np.abs(sk).max()))
                worst = max(worst, e)
                assert e <= 1e-12, f"gradient sums off by {e}"
    return worst


def pin_groups(bwd):
    rng = np.random.default_rng(24)
    B, T, Hq, Hkv, d, L_d = 2, 6, 6, 2, 5, 3
    *x, dout = _inputs(rng, B, T, Hq, Hkv, d, L_d)
    dq, _, _, dkd, dvd = bwd(*x, dout)
    G = Hq // Hkv
    groups = [(1, 5, 1), (0, 0, 0), (1, 2, 0)]
    gq, gkd, gvd = bwd(*x, dout, groups=groups)
    worst = 0.0
    for i, (b, t, kvh) in enumerate(groups):
        e = max(float(np.abs(gq[i] - dq[b, t, kvh * G:(kvh + 1) * G]).max()),
                float(np.abs(gkd[i] - dkd[b, t, :, kvh]).max()),
                float(np.abs(gvd[i] - dvd[b, t, :, kvh]).max()))
        worst = max(worst, e)
        assert e <= 1e-13, f"group {(b, t, kvh)}: {e}"
    return worst


def pin_keys(keys_fn, bwd=None):
    """keys_fn has the signature of oracle.moda_backward_keys; the full form
    comes from `bwd` (default: the oracle's moda_backward)."""
    if bwd is None:
        from oracle import moda_backward as bwd
    rng = np.random.default_rng(25)
    worst = 0.0
    for (B, T, Hq, Hkv, d, L_d) in [(2, 9, 6, 2, 5, 3), (1, 7, 2, 2, 4, 0), (1, 6, 4, 1, 3, 2)]:
        *x, dout = _inputs(rng, B, T, Hq, Hkv, d, L_d)
        _, dks, dvs, _, _ = bwd(*x, dout)
        keys = [(b, s, kvh) for b in range(B) for s in range(T) for kvh in range(Hkv)]
        gk, gv = keys_fn(*x, dout, keys=keys)
        for i, (b, s, kvh) in enumerate(keys):
            e = max(float(np.abs(gk[i] - dks[b, s, kvh]).max()), float(np.abs(gv[i] - dvs[b, s, kvh]).max()))
            worst = max(worst, e)
            assert e <= 1e-12, f"key {(b, s, kvh)} of shape {(B, T, Hq, Hkv, d, L_d)}: {e}"
    return worst


BWD_PINS = {
    "finite_diff": pin_finite_diff,
    "autograd": pin_autograd,
    "sums": pin_sums,
    "groups": pin_groups,
}
