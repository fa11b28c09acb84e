"""Oracle for the Mixture-of-Depths Attention (MoDA) forward pass.

TEST INFRASTRUCTURE ONLY.  This module is the slow, plain, obviously correct
CPU definition that the GPU kernels are checked against.  Only the tests, the
smoke check and the CPU-baseline leg of the benchmark may import it; the
product path never does, and this module imports nothing from the product.

What is computed (exact attention, evaluated in float64):

  For query position t of head h (batch b) the key set is the concatenation of
    * the causal sequence keys of the current layer, positions s = 0..t, and
    * the L_d depth keys that earlier layers wrote for the SAME position t,
  and one softmax, scaled by 1/sqrt(d), runs over the whole concatenation; the
  output is the matching weighted sum of values.

  Sources (all pages are summaries of arXiv 2603.15619, "Mixture-of-Depths
  Attention"):
    * mhpn.cn article "动态混合深度注意力机制MoDA技术解析", section 1.2: the MoDA
      attention formula -- softmax over [Q K_l^T || Q K_{l-1}^T || ... ||
      Q K_0^T] / sqrt(d), times the concatenated values.
    * same article, section 2.2 ("双重掩码机制"): the sequence mask lets a token
      see itself and earlier positions; the depth mask lets a query see only the
      depth history of its own position (prevents information leakage).
    * gist.science (de) "Mixture-of-Depths Attention", Technische
      Zusammenfassung section 2, Kernkonzept: Read-Step (same position t, all
      earlier layers) and Unified Softmax (one normalisation for both sets).
    * gist.science (de), same section, Group-Aware Indexing: GQA, several
      query heads share one KV head.

Readings taken where the pages leave a step open:
    * the formula's Q K_i^T terms are taken before masking; the depth mask
      restricts them to position t;
    * the causal mask includes s = t ("itself and earlier");
    * the same 1/sqrt(d) scale applies to depth scores (the formula divides the
      whole concatenation);
    * GQA head map: query head h uses KV head h // G with G = Hq / Hkv;
    * layouts: q/out [B,T,Hq,d], k/v_seq [B,T,Hkv,d], depth [B,T,L_d,Hkv,d],
      lse [B,Hq,T];
    * lse is the natural log of the sum of exp of the scaled scores.

Parity pins: every function here is pinned by the CPU tests in
tests/test_oracle_pins.py (library special cases, closed forms, invariants and
brute force); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype != np.float64:
        a = a.astype(np.float64)
    return a


def _check_shapes(q, k_seq, v_seq, k_depth, v_depth):
    if q.ndim != 4:
        raise ValueError("q must be [B,T,Hq,d]")
    B, T, Hq, d = q.shape
    if k_seq.ndim != 4 or k_seq.shape[:2] != (B, T) or k_seq.shape[3] != d:
        raise ValueError("k_seq must be [B,T,Hkv,d]")
    Hkv = k_seq.shape[2]
    if v_seq.shape != k_seq.shape:
        raise ValueError("v_seq must match k_seq")
    if Hkv < 1 or Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if k_depth.ndim != 5 or k_depth.shape[:2] != (B, T) or k_depth.shape[3:] != (Hkv, d):
        raise ValueError("k_depth must be [B,T,L_d,Hkv,d]")
    if v_depth.shape != k_depth.shape:
        raise ValueError("v_depth must match k_depth")
    return B, T, Hq, Hkv, d, k_depth.shape[2]


def moda_forward(q, k_seq, v_seq, k_depth, v_depth,
                 rows: Optional[Sequence[Sequence[int]]] = None,
                 return_probs: bool = False):
    """MoDA forward by its definition, in float64.

    Arguments are array-likes (converted exactly to float64):
      q [B,T,Hq,d], k_seq/v_seq [B,T,Hkv,d], k_depth/v_depth [B,T,L_d,Hkv,d]
      (L_d may be 0).

    rows: optional list of (b, t, h) triples.  With rows=None the full output
    is returned as (out [B,T,Hq,d], lse [B,Hq,T]); with rows given, as
    (out [n,d], lse [n]) in the order of `rows`.

    return_probs: also return, per computed row, the probability vector over
    the concatenated key set (sequence keys 0..t first, then depth slots
    0..L_d-1).  Only meant for tiny shapes.

    One (b, t, kv-head) group at a time: the G query rows of that group are
    scored against the concatenated key set
        [k_seq[b, 0..t, kvh] ; k_depth[b, t, 0..L_d-1, kvh]]
    (mhpn.cn article, section 1.2 formula; section 2.2 masks) as the
    concatenation of the two score blocks, the scores are scaled by 1/sqrt(d),
    and a single softmax is taken over all of them (gist.science (de),
    section 2, Unified Softmax).
    """
    q = np.asarray(q)
    k_seq = np.asarray(k_seq)
    v_seq = np.asarray(v_seq)
    k_depth = np.asarray(k_depth)
    v_depth = np.asarray(v_depth)
    B, T, Hq, Hkv, d, L_d = _check_shapes(q, k_seq, v_seq, k_depth, v_depth)
    G = Hq // Hkv
    scale = 1.0 / math.sqrt(d)
    # Sequence keys / values of each (b, kv head) as contiguous float64
    # [B, Hkv, T, d] (an exact conversion; only the layout changes), so that
    # the prefix 0..t of one head is a plain contiguous slice.
    Kseq = _f64(np.ascontiguousarray(np.transpose(k_seq, (0, 2, 1, 3))))
    Vseq = _f64(np.ascontiguousarray(np.transpose(v_seq, (0, 2, 1, 3))))

    if rows is None:
        groups = {}
        for b in range(B):
            for t in range(T):
                for kvh in range(Hkv):
                    groups[(b, t, kvh)] = list(range(kvh * G, (kvh + 1) * G))
    else:
        rows = [tuple(int(x) for x in r) for r in rows]
        groups = {}
        for (b, t, h) in rows:
            if not (0 <= b < B and 0 <= t < T and 0 <= h < Hq):
                raise ValueError(f"row {(b, t, h)} out of range")
            groups.setdefault((b, t, h // G), [])
            if h not in groups[(b, t, h // G)]:
                groups[(b, t, h // G)].append(h)

    res_out = {}
    res_lse = {}
    res_p = {}
    for (b, t, kvh), heads in groups.items():
        # The key set of position t: sequence keys s = 0..t of this layer
        # (causal mask), then the L_d depth slots of position t itself
        # (depth mask).
        Ks = Kseq[b, kvh, : t + 1]                  # [t+1, d]
        Vs = Vseq[b, kvh, : t + 1]
        Kd = _f64(k_depth[b, t, :, kvh, :])         # [L_d, d]
        Vd = _f64(v_depth[b, t, :, kvh, :])
        Qg = _f64(q[b, t, heads, :])                # [g, d]
        # Scores: the concatenation [Q K_seq^T || Q K_depth^T], scaled by
        # 1/sqrt(d) as a whole (mhpn.cn article, section 1.2 formula).
        z = np.concatenate([Qg @ Ks.T, Qg @ Kd.T], axis=1) * scale   # [g, t+1+L_d]
        # One softmax over the whole concatenation (Unified Softmax).
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        Z = e.sum(axis=1, keepdims=True)
        p = e / Z
        # p times the concatenated values [V_seq ; V_depth]: the product with
        # a concatenation is the sum of the two block products.
        ns = t + 1
        o = p[:, :ns] @ Vs + p[:, ns:] @ Vd         # [g, d]
        lse = m[:, 0] + np.log(Z[:, 0])
        for i, h in enumerate(heads):
            res_out[(b, t, h)] = o[i]
            res_lse[(b, t, h)] = lse[i]
            if return_probs:
                res_p[(b, t, h)] = p[i]

    if rows is None:
        out = np.empty((B, T, Hq, d), dtype=np.float64)
        lse = np.empty((B, Hq, T), dtype=np.float64)
        for (b, t, h), o in res_out.items():
            out[b, t, h] = o
            lse[b, h, t] = res_lse[(b, t, h)]
        if return_probs:
            return out, lse, res_p
        return out, lse
    out = np.stack([res_out[r] for r in rows]) if rows else np.zeros((0, d))
    lse = np.array([res_lse[r] for r in rows], dtype=np.float64)
    if return_probs:
        return out, lse, [res_p[r] for r in rows]
    return out, lse


def moda_forward_scalar(q, k_seq, v_seq, k_depth, v_depth):
    """The same definition with scalar Python loops, for tiny shapes only.

    Written independently of `moda_forward` (no numpy arithmetic): scores are
    plain dot products, the exponentials use math.exp, sums use math.fsum.
    Inputs are nested lists or arrays with the layouts of `moda_forward`.
    Returns (out, lse) as nested Python lists [B][T][Hq][d] and [B][Hq][T].
    """
    q = np.asarray(q, dtype=np.float64).tolist()
    k_seq = np.asarray(k_seq, dtype=np.float64).tolist()
    v_seq = np.asarray(v_seq, dtype=np.float64).tolist()
    k_depth = np.asarray(k_depth, dtype=np.float64)
    L_d = k_depth.shape[2]
    k_depth = k_depth.tolist()
    v_depth = np.asarray(v_depth, dtype=np.float64).tolist()
    B = len(q)
    T = len(q[0])
    Hq = len(q[0][0])
    d = len(q[0][0][0])
    Hkv = len(k_seq[0][0])
    G = Hq // Hkv
    out = [[[[0.0] * d for _ in range(Hq)] for _ in range(T)] for _ in range(B)]
    lse = [[[0.0] * T for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for t in range(T):
            for h in range(Hq):
                kvh = h // G
                qv = q[b][t][h]
                keys = [k_seq[b][s][kvh] for s in range(t + 1)]
                vals = [v_seq[b][s][kvh] for s in range(t + 1)]
                keys += [k_depth[b][t][j][kvh] for j in range(L_d)]
                vals += [v_depth[b][t][j][kvh] for j in range(L_d)]
                scores = [math.fsum(qv[i] * kk[i] for i in range(d)) / math.sqrt(d)
                          for kk in keys]
                mx = max(scores)
                ex = [math.exp(s - mx) for s in scores]
                Z = math.fsum(ex)
                for i in range(d):
                    out[b][t][h][i] = math.fsum(ex[j] * vals[j][i] for j in range(len(vals))) / Z
                lse[b][h][t] = mx + math.log(Z)
    return out, lse


def depth_utilisation(C: int, G: int, L: int, T: int, layout: str) -> float:
    """Share of computed depth scores that the depth mask keeps.

    Counts mask entries one by one (mhpn.cn article, section 2.2 and its
    Figure 4 discussion of the depth-KV layout):
      * layout "naive": every query row scores the whole flattened T x L
        depth axis; a row at position t keeps only the L slots of t.
      * layout "chunked": query rows are taken in chunks of C rows; with GQA,
        G adjacent rows share one position, so a chunk covers C / G positions
        and scores only those positions' C / G * L depth keys.
    Rows are (position, head-in-group) pairs, position-major.  For the chunked
    layout G must divide C and C / G must divide T.
    """
    if layout == "naive":
        kept = 0
        computed = 0
        for r in range(T * G):
            t = r // G
            for n in range(T * L):
                computed += 1
                kept += (n // L == t)
        return kept / computed
    if layout == "chunked":
        if C % G != 0 or T % (C // G) != 0:
            raise ValueError("chunked layout needs G | C and (C/G) | T")
        P = C // G
        kept = 0
        computed = 0
        for c0 in range(0, T * G, C):
            t_first = c0 // G
            keys = [(t_first + p) * L + j for p in range(P) for j in range(L)]
            for r in range(c0, c0 + C):
                t = r // G
                for n in keys:
                    computed += 1
                    kept += (n // L == t)
        return kept / computed
    raise ValueError(f"unknown layout {layout!r}")
