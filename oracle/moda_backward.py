"""Oracle for the gradients of the Mixture-of-Depths Attention (MoDA) forward.

TEST INFRASTRUCTURE ONLY, like oracle/moda_oracle.py: the slow, plain CPU
definition that the GPU backward kernels are checked against.  Only the tests,
the smoke check and the CPU-baseline leg of the benchmark may import it; the
product never does, and it imports nothing from the product.

What is computed.  The forward is the concatenated-set softmax of the mhpn.cn
article "动态混合深度注意力机制MoDA技术解析", section 1.2 (MoDA attention
formula), with the causal and same-position depth masks of section 2.2: for
each (b, t, h), with kv head kvh = h // G,
    z   = [q . k_seq[b, s, kvh] for s <= t ; q . k_depth[b, t, j, kvh] for all j] / sqrt(d)
    p   = softmax(z)
    out = p . [v_seq[b, 0..t, kvh] ; v_depth[b, t, :, kvh]]
The pages do not write out a backward pass; they present the kernel as usable
in training pipelines (gist.science (de) "Mixture-of-Depths Attention",
section 5, Praktische Anwendbarkeit).  The gradients here are the derivatives
of that forward for a loss L whose gradient with respect to out is `dout`,
by the chain rule through the three steps above:
    dL/dv_j    = sum over the rows that see key j of  p_j * dout
    dL/dp_j    = dout . v_j
    dL/dz_j    = p_j * (dL/dp_j - sum_i p_i * dL/dp_i)        (softmax Jacobian)
    dL/dq      = (1/sqrt(d)) * sum_j dL/dz_j * k_j
    dL/dk_j    = (1/sqrt(d)) * sum over the rows that see key j of  dL/dz_j * q
Key j is a sequence key s (seen by every row at a position >= s, all G heads of
its kv head) or a depth slot of position t (seen only by the G heads at t), so
the sequence gradients sum over positions and heads, the depth gradients over
the G heads of one position.

Parity pins (tests/test_oracle_backward.py): central finite differences of the
forward oracle, torch autograd of float64 masked attention (a library routine)
with and without depth, the exact sums sum_j dL/dv_j = sum_i dout_i and
sum_j dL/dk_j = 0 per kv head, the sampled-group form against the full form,
and the per-key form (moda_backward_keys) against the full form.  None of
these functions is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _group_grads(Qg, dOg, Ks, Vs, Kd, Vd, scale):
    """Gradients of one (b, t, kv-head) group: the g query rows of position t
    against its concatenated key set [Ks ; Kd] (sequence keys 0..t, then the
    depth slots of t).  Returns dQ [g,d], dKs, dVs [t+1,d], dKd, dVd [L_d,d]."""
    Kc = np.concatenate([Ks, Kd], axis=0)          # [n, d]
    Vc = np.concatenate([Vs, Vd], axis=0)
    z = (Qg @ Kc.T) * scale                        # [g, n]
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    p = e / e.sum(axis=1, keepdims=True)
    dV = p.T @ dOg                                 # [n, d]
    dp = dOg @ Vc.T                                # [g, n]
    dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dQ = (dz @ Kc) * scale                         # [g, d]
    dK = (dz.T @ Qg) * scale                       # [n, d]
    ns = Ks.shape[0]
    return dQ, dK[:ns], dV[:ns], dK[ns:], dV[ns:]


def moda_backward(q, k_seq, v_seq, k_depth, v_depth, dout,
                  groups: Optional[Sequence[tuple]] = None):
    """Gradients of the MoDA forward, float64.

    Layouts as in oracle.moda_forward: q, dout [B,T,Hq,d]; k_seq, v_seq
    [B,T,Hkv,d]; k_depth, v_depth [B,T,L_d,Hkv,d] (L_d may be 0).

    groups=None: returns the full gradients
        (dq [B,T,Hq,d], dk_seq [B,T,Hkv,d], dv_seq [B,T,Hkv,d],
         dk_depth [B,T,L_d,Hkv,d], dv_depth [B,T,L_d,Hkv,d]).
    groups = list of (b, t, kvh): returns, in that order, the gradients that
    depend on that group alone,
        (dq [n,G,d] for heads kvh*G .. kvh*G+G-1 at (b, t),
         dk_depth [n,L_d,d], dv_depth [n,L_d,d] of slots of (b, t, kvh)),
    since a depth slot is seen only by the G heads of its own position and a
    query row sees only its own group's key set.  Sequence-key gradients sum
    over all later positions and are returned only in the full form.
    """
    q, k_seq, v_seq = np.asarray(q), np.asarray(k_seq), np.asarray(v_seq)
    k_depth, v_depth, dout = np.asarray(k_depth), np.asarray(v_depth), np.asarray(dout)
    B, T, Hq, d = q.shape
    Hkv = k_seq.shape[2]
    L_d = k_depth.shape[2]
    if Hq % Hkv or k_seq.shape != (B, T, Hkv, d) or v_seq.shape != k_seq.shape:
        raise ValueError("inconsistent sequence shapes")
    if k_depth.shape != (B, T, L_d, Hkv, d) or v_depth.shape != k_depth.shape:
        raise ValueError("inconsistent depth shapes")
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    Kseq = _f64(np.transpose(k_seq, (0, 2, 1, 3)))  # [B, Hkv, T, d]
    Vseq = _f64(np.transpose(v_seq, (0, 2, 1, 3)))

    def group(b, t, kvh):
        heads = slice(kvh * G, (kvh + 1) * G)
        return _group_grads(_f64(q[b, t, heads]), _f64(dout[b, t, heads]),
                            Kseq[b, kvh, : t + 1], Vseq[b, kvh, : t + 1],
                            _f64(k_depth[b, t, :, kvh]), _f64(v_depth[b, t, :, kvh]), scale)

    if groups is not None:
        n = len(groups)
        dq = np.zeros((n, G, d))
        dkd = np.zeros((n, L_d, d))
        dvd = np.zeros((n, L_d, d))
        for i, (b, t, kvh) in enumerate(groups):
            if not (0 <= b < B and 0 <= t < T and 0 <= kvh < Hkv):
                raise ValueError(f"group {(b, t, kvh)} out of range")
            gq, _, _, gkd, gvd = group(b, t, kvh)
            dq[i], dkd[i], dvd[i] = gq, gkd, gvd
        return dq, dkd, dvd

    dq = np.zeros((B, T, Hq, d))
    dks = np.zeros((B, Hkv, T, d))
    dvs = np.zeros((B, Hkv, T, d))
    dkd = np.zeros((B, T, L_d, Hkv, d))
    dvd = np.zeros((B, T, L_d, Hkv, d))
    for b in range(B):
        for t in range(T):
            for kvh in range(Hkv):
                gq, gks, gvs, gkd, gvd = group(b, t, kvh)
                dq[b, t, kvh * G:(kvh + 1) * G] = gq
                dks[b, kvh, : t + 1] += gks
                dvs[b, kvh, : t + 1] += gvs
                dkd[b, t, :, kvh] = gkd
                dvd[b, t, :, kvh] = gvd
    return (dq, np.transpose(dks, (0, 2, 1, 3)).copy(), np.transpose(dvs, (0, 2, 1, 3)).copy(),
            dkd, dvd)


def moda_backward_keys(q, k_seq, v_seq, k_depth, v_depth, dout, keys: Sequence[tuple]):
    """Gradients of selected sequence keys, one key (column) at a time.

    keys = list of (b, s, kvh).  Returns (dk [n,d], dv [n,d]) in that order:
    dL/dk_seq[b, s, kvh] and dL/dv_seq[b, s, kvh], float64.

    The same derivative as moda_backward, written per key instead of per query
    group.  Sequence key s of kv head kvh is seen by every row (b, t, h) with
    t >= s (the causal mask of the mhpn.cn article, section 2.2) and h one of
    the G query heads of kvh.  For such a row, with its lse and out from the
    forward oracle,
        p     = exp(q_row . k_s / sqrt(d) - lse_row)        (its weight on s)
        Delta = dout_row . out_row   (= sum_j p_j dL/dp_j, because
                                      out_row = sum_j p_j v_j)
        dL/dv_s += p * dout_row
        dL/dk_s += p * (dout_row . v_s - Delta) * q_row / sqrt(d)
    Only the rows at positions s .. T-1 of the key's own (b, kv head) are
    evaluated, so the cost is bounded for keys near the end of a long
    sequence.
    """
    from .moda_oracle import moda_forward

    q, k_seq, v_seq = np.asarray(q), np.asarray(k_seq), np.asarray(v_seq)
    dout = np.asarray(dout)
    B, T, Hq, d = q.shape
    Hkv = k_seq.shape[2]
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    keys = [tuple(int(x) for x in k) for k in keys]
    for (b, s, kvh) in keys:
        if not (0 <= b < B and 0 <= s < T and 0 <= kvh < Hkv):
            raise ValueError(f"key {(b, s, kvh)} out of range")
    # every row that sees at least one selected key: per (b, kv head), the
    # positions from the earliest selected key to the end, all G heads
    first = {}
    for (b, s, kvh) in keys:
        first[(b, kvh)] = min(s, first.get((b, kvh), T))
    rows = [(b, t, h) for (b, kvh), s0 in sorted(first.items())
            for t in range(s0, T) for h in range(kvh * G, (kvh + 1) * G)]
    out, lse = moda_forward(q, k_seq, v_seq, k_depth, v_depth, rows=rows)
    at = {r: i for i, r in enumerate(rows)}
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    for n, (b, s, kvh) in enumerate(keys):
        ks_ = _f64(k_seq[b, s, kvh])
        vs_ = _f64(v_seq[b, s, kvh])
        idx = [at[(b, t, h)] for t in range(s, T) for h in range(kvh * G, (kvh + 1) * G)]
        Qr = _f64(q[b, s:, kvh * G:(kvh + 1) * G]).reshape(-1, d)      # rows (t, h), t-major
        dOr = _f64(dout[b, s:, kvh * G:(kvh + 1) * G]).reshape(-1, d)
        p = np.exp((Qr @ ks_) * scale - lse[idx])
        delta = (dOr * out[idx]).sum(axis=1)
        dv[n] = p @ dOr
        dk[n] = ((p * (dOr @ vs_ - delta)) @ Qr) * scale
    return dk, dv
