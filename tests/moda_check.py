"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same seeded inputs, compare element by element."""
from __future__ import annotations

import numpy as np
import torch

import depth_augmented_attention_amd as moda
from oracle import moda_backward_keys, moda_forward

# Tolerances on max |gpu - oracle| (out and lse), by input dtype: float32
# inputs are computed in float32 end to end; bf16 inputs use bf16 matrix-core
# products with float32 accumulation, bf16 probabilities in the P.V product
# and a bf16-rounded output.
TOL = {torch.float32: 1e-5, torch.bfloat16: 1.5e-2}


def np32(x: torch.Tensor) -> np.ndarray:
    """Exact float32 numpy copy of a CPU tensor (bf16 values are exact in fp32)."""
    return x.detach().to("cpu").to(torch.float32).numpy()


def run_gpu(q, k_seq, v_seq, k_depth, v_depth, with_lse=True, stream=None):
    """Pack + fused forward on cuda:0 for CPU input tensors; returns GPU tensors."""
    dev = torch.device("cuda:0")
    L_d = k_depth.shape[2]
    qd, kd_, vd_ = q.to(dev), k_seq.to(dev), v_seq.to(dev)
    if L_d > 0:
        kp, vp = moda.moda_pack_depth(k_depth.to(dev), v_depth.to(dev), stream=stream)
    else:
        kp = vp = None
    out, lse = moda.moda_fwd(qd, kd_, vd_, kp, vp, L_d, with_lse=with_lse, stream=stream)
    torch.cuda.synchronize()
    return out, lse


def compare_all_rows(inputs, out, lse):
    """Full-output comparison; returns (max err out, max err lse)."""
    ref_out, ref_lse = moda_forward(*[np32(x) for x in inputs])
    o = out.detach().to("cpu").to(torch.float64).numpy()
    err_o = float(np.abs(o - ref_out).max())
    err_l = float(np.abs(lse.detach().cpu().double().numpy() - ref_lse).max()) if lse is not None else 0.0
    return err_o, err_l


def compare_rows(inputs, out, lse, rows):
    """Comparison on sampled (b, t, h) rows; returns (max err out, max err lse)."""
    ref_out, ref_lse = moda_forward(*[np32(x) for x in inputs], rows=rows)
    rows = np.asarray(rows)
    b, t, h = rows[:, 0], rows[:, 1], rows[:, 2]
    bt = torch.from_numpy(b).to(out.device)
    tt = torch.from_numpy(t).to(out.device)
    ht = torch.from_numpy(h).to(out.device)
    o = out[bt, tt, ht].to(torch.float64).cpu().numpy()
    err_o = float(np.abs(o - ref_out).max())
    err_l = 0.0
    if lse is not None:
        l = lse[bt, ht, tt].to(torch.float64).cpu().numpy()
        err_l = float(np.abs(l - ref_lse).max())
    return err_o, err_l


def rel_err(got, ref):
    """max |got - ref| / max(1, max |ref|): the backward's error measure (sums
    over many rows, such as the gradients of early keys, grow with T)."""
    if ref.size == 0:
        return 0.0
    return float(np.abs(got - ref).max()) / max(1.0, float(np.abs(ref).max()))


def tail_keys(T, last=64, bounds=(128, 256)):
    """Sequence keys checked element by element at large T: the last `last`
    keys (the last key tiles and query-row blocks of the dK/dV kernel, at its
    highest offsets) and the keys on each side of the 128-key tile
    boundaries T - 128 and T - 256 (and of T rounded down to those tiles)."""
    ks = set(range(max(0, T - last), T))
    for bnd in bounds:
        for edge in (T - bnd, (T - 1) // 128 * 128 - (bnd - 128)):
            ks |= {edge - 1, edge}
    return sorted(s for s in ks if 0 <= s < T)


def key_errors(tag, q, ks, vs, kd, vd, dout, dks_gpu, dvs_gpu, B, Hkv, keys_s):
    """max |gpu - oracle| / max(1, max |oracle|) of dk_seq and dv_seq at the
    given keys of every (b, kv head), against the oracle's per-key form.
    dks_gpu / dvs_gpu: [B,T,Hkv,d] GPU tensors (or arrays)."""
    keys = [(b, s, kvh) for b in range(B) for s in keys_s for kvh in range(Hkv)]
    rk, rv = moda_backward_keys(q, ks, vs, kd, vd, dout, keys=keys)
    sel = lambda g: np.stack([(g[b, s, kvh].double().cpu().numpy() if torch.is_tensor(g) else g[b, s, kvh])
                              for (b, s, kvh) in keys])
    return {f"dk_seq[{tag}]": rel_err(sel(dks_gpu), rk), f"dv_seq[{tag}]": rel_err(sel(dvs_gpu), rv)}
