"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no attention arithmetic: it only draws the i.i.d. N(0, 1)
tensors (rounded to bf16 for the bf16 workloads), lists the workload shapes and
picks the sampled query rows that large workloads are checked on.  Both the
GPU path and the oracle consume what it returns.

Recipe: one CPU torch.Generator seeded with the workload's seed draws, in this
order, q [B,T,Hq,d], k_seq [B,T,Hkv,d], v_seq [B,T,Hkv,d],
k_depth [B,T,L_d,Hkv,d], v_depth [B,T,L_d,Hkv,d] as float32 standard normals;
bf16 workloads then round each to bf16 (round to nearest even).
"""
from __future__ import annotations

import numpy as np
import torch

# The workloads.  The pages benchmark at sequence lengths 4K..64K and at GQA
# group sizes 8 and 32 (mhpn.cn article, section 3.1, Table 2 discussion);
# head counts, head size and depth are chosen here (the pages do not state
# them).
WORKLOADS = [
    dict(name="fp32_B1_T128_Hq4_Hkv1_d64_L3", dtype="fp32", B=1, T=128, Hq=4, Hkv=1, d=64, L_d=3, seed=1001),
    dict(name="bf16_B1_T4096_Hq16_Hkv2_d128_L24", dtype="bf16", B=1, T=4096, Hq=16, Hkv=2, d=128, L_d=24, seed=1002),
    dict(name="bf16_B2_T16384_Hq16_Hkv2_d128_L24", dtype="bf16", B=2, T=16384, Hq=16, Hkv=2, d=128, L_d=24, seed=1003),
    dict(name="bf16_B1_T65536_Hq16_Hkv2_d128_L24", dtype="bf16", B=1, T=65536, Hq=16, Hkv=2, d=128, L_d=24, seed=1004),
    dict(name="bf16_B1_T65536_Hq32_Hkv1_d128_L48", dtype="bf16", B=1, T=65536, Hq=32, Hkv=1, d=128, L_d=48, seed=1005),
]


def workload(name: str) -> dict:
    for w in WORKLOADS:
        if w["name"] == name:
            return dict(w)
    raise KeyError(name)


def torch_dtype(dtype: str) -> torch.dtype:
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[dtype]


def make_inputs(B, T, Hq, Hkv, d, L_d, dtype="bf16", seed=0, depth=True):
    """Draw (q, k_seq, v_seq, k_depth, v_depth) as CPU tensors of `dtype`.

    With depth=False the two depth tensors are not drawn (returned as empty
    [B,T,0,Hkv,d] tensors); the first three are the same as with depth=True.
    """
    g = torch.Generator().manual_seed(int(seed))
    td = torch_dtype(dtype)

    def draw(*shape):
        x = torch.randn(*shape, generator=g, dtype=torch.float32)
        return x if td == torch.float32 else x.to(td)

    q = draw(B, T, Hq, d)
    k_seq = draw(B, T, Hkv, d)
    v_seq = draw(B, T, Hkv, d)
    if depth and L_d > 0:
        k_depth = draw(B, T, L_d, Hkv, d)
        v_depth = draw(B, T, L_d, Hkv, d)
    else:
        k_depth = torch.empty(B, T, 0, Hkv, d, dtype=td)
        v_depth = torch.empty(B, T, 0, Hkv, d, dtype=td)
    return q, k_seq, v_seq, k_depth, v_depth


def make_dout(B, T, Hq, d, dtype="bf16", seed=0):
    """Draw the gradient of the output, [B,T,Hq,d] N(0,1) of `dtype`, from its
    own generator (seed + 500) so that the forward inputs are unchanged."""
    g = torch.Generator().manual_seed(int(seed) + 500)
    x = torch.randn(B, T, Hq, d, generator=g, dtype=torch.float32)
    td = torch_dtype(dtype)
    return x if td == torch.float32 else x.to(td)


def make_workload_inputs(w: dict, depth=True):
    return make_inputs(w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"],
                       dtype=w["dtype"], seed=w["seed"], depth=depth)


def to_f64(x) -> np.ndarray:
    """Exact conversion of a CPU tensor (fp32 or bf16) to a float64 array."""
    return x.detach().to("cpu").to(torch.float64).numpy()


def sample_rows(B, T, Hq, n=4096, seed=0, tile_rows=()):
    """Distinct (b, t, h) query rows to check a large output on.

    Draws n distinct flat row indices with numpy's default_rng(seed), then adds
    the first row, the last row and, for each position in `tile_rows`, the
    first and last head of that position (used for tile boundaries).
    """
    total = B * T * Hq
    rng = np.random.default_rng(int(seed))
    n = min(n, total)
    flat = rng.choice(total, size=n, replace=False)
    rows = {(int(f // (T * Hq)), int((f // Hq) % T), int(f % Hq)) for f in flat}
    rows.add((0, 0, 0))
    rows.add((B - 1, T - 1, Hq - 1))
    for t in tile_rows:
        if 0 <= t < T:
            rows.add((B // 2, t, 0))
            rows.add((B // 2, t, Hq - 1))
    return np.array(sorted(rows), dtype=np.int64)
