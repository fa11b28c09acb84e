"""GPU parity: the HIP path (through the C ABI) against the oracle.

Every case prints what it runs before touching the GPU.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import depth_augmented_attention_amd as moda
from moda_check import TOL, compare_all_rows, compare_rows, np32, run_gpu
from moda_inputs import WORKLOADS, make_inputs, make_workload_inputs, sample_rows

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _check(name, dtype, err_o, err_l):
    tol = TOL[dtype]
    _say(f"{name}: max|out-ref| = {err_o:.3e}  max|lse-ref| = {err_l:.3e}  (tol {tol:g})")
    assert err_o <= tol, f"{name}: out error {err_o} > {tol}"
    assert err_l <= tol, f"{name}: lse error {err_l} > {tol}"


SMALL = [w for w in WORKLOADS if w["T"] <= 4096]
LARGE = [w for w in WORKLOADS if w["T"] > 4096]


@pytest.mark.parametrize("w", SMALL, ids=[w["name"] for w in SMALL])
def test_workload_all_rows(w):
    _say(f"workload {w['name']} (all rows)")
    inputs = make_workload_inputs(w)
    out, lse = run_gpu(*inputs)
    _check(w["name"], inputs[0].dtype, *compare_all_rows(inputs, out, lse))


@pytest.mark.parametrize("w", LARGE, ids=[w["name"] for w in LARGE])
def test_workload_sampled_rows(w):
    _say(f"workload {w['name']} (4096 sampled rows)")
    inputs = make_workload_inputs(w)
    G = w["Hq"] // w["Hkv"]
    P = 128 // G if G <= 128 else 1        # positions per 128-row query tile
    mid = (w["T"] // 2) // P * P
    rows = sample_rows(w["B"], w["T"], w["Hq"], n=4096, seed=w["seed"] + 7,
                       tile_rows=(mid, mid + P - 1, w["T"] - 1))
    out, lse = run_gpu(*inputs)
    _check(w["name"], inputs[0].dtype, *compare_rows(inputs, out, lse, rows))
    if w["T"] == 65536 and w["Hkv"] == 2:
        # the same q / k_seq / v_seq without depth slots (plain causal GQA)
        _say(f"workload {w['name']} at L_d = 0")
        q, ks, vs = inputs[:3]
        empty = torch.empty(w["B"], w["T"], 0, w["Hkv"], w["d"], dtype=q.dtype)
        out0, lse0 = run_gpu(q, ks, vs, empty, empty)
        _check(w["name"] + " L_d=0", q.dtype, *compare_rows((q, ks, vs, empty, empty), out0, lse0, rows))


EDGE = [
    # dtype, B, T, Hq, Hkv, d, L_d
    ("bf16", 1, 1, 4, 1, 128, 0),      # single position, no depth
    ("bf16", 1, 1, 4, 1, 128, 3),      # single position with depth
    ("fp32", 1, 1, 2, 2, 64, 0),
    ("bf16", 3, 77, 6, 3, 128, 5),     # ragged T, T*L_d not a multiple of 32
    ("bf16", 2, 333, 8, 8, 64, 7),     # G = 1
    ("fp32", 1, 200, 32, 1, 128, 2),   # G = 32, float32, d = 128
    ("bf16", 1, 1000, 12, 1, 128, 1),  # G = 12 (rows of a position straddle waves)
    ("bf16", 1, 129, 2, 1, 128, 33),   # L_d > 32
    ("fp32", 2, 65, 3, 1, 64, 4),      # G = 3
    ("bf16", 1, 300, 64, 1, 128, 2),   # G = 64 > 32 rows of a wave
    ("fp32", 1, 130, 4, 1, 64, 0),     # depth-free float32 with a ragged last block
    # grids large enough for the eight-wave (256-row) bf16 tiles, ragged tails
    ("bf16", 4, 1100, 32, 16, 128, 3), # G = 2, 9 tiles of 256 rows x 64 (b, kv head)
    ("bf16", 2, 2100, 64, 16, 128, 5), # G = 4, ragged last tile, L_d * T not a multiple of 32
]


@pytest.mark.parametrize("case", EDGE, ids=[
    f"{c[0]}_B{c[1]}_T{c[2]}_Hq{c[3]}_Hkv{c[4]}_d{c[5]}_L{c[6]}" for c in EDGE])
def test_edge_shapes(case):
    dtype, B, T, Hq, Hkv, d, L_d = case
    _say(f"edge case {case}")
    inputs = make_inputs(B, T, Hq, Hkv, d, L_d, dtype=dtype, seed=77 + T + L_d)
    out, lse = run_gpu(*inputs)
    _check(str(case), inputs[0].dtype, *compare_all_rows(inputs, out, lse))


def _pack_reference(kd: np.ndarray, vd: np.ndarray):
    """The packed layout written out from its documented definition."""
    B, T, L_d, Hkv, d = kd.shape
    n = T * L_d
    NKp = (n + 31) // 32 * 32
    kp = np.zeros((B, Hkv, NKp, d), dtype=kd.dtype)
    vp = np.zeros((B, Hkv, NKp, d), dtype=vd.dtype)
    kp[:, :, :n] = np.transpose(kd, (0, 3, 1, 2, 4)).reshape(B, Hkv, n, d)
    vp[:, :, :n] = np.transpose(vd, (0, 3, 1, 2, 4)).reshape(B, Hkv, n, d)
    return kp.reshape(-1), vp.reshape(-1)


@pytest.mark.parametrize("case", [("bf16", 2, 37, 3, 128, 5), ("fp32", 1, 64, 2, 64, 3), ("bf16", 1, 40, 1, 64, 24)])
def test_pack_layout_bitwise(case):
    dtype, B, T, Hkv, d, L_d = case
    _say(f"pack layout {case}")
    _, _, _, kd, vd = make_inputs(B, T, Hkv, Hkv, d, L_d, dtype=dtype, seed=5)
    kp, vp = moda.moda_pack_depth(kd.cuda(), vd.cuda())
    torch.cuda.synchronize()
    view = torch.int16 if dtype == "bf16" else torch.int32
    rk, rv = _pack_reference(kd.view(view).numpy(), vd.view(view).numpy())
    assert np.array_equal(kp.cpu().view(view).numpy(), rk)
    assert np.array_equal(vp.cpu().view(view).numpy(), rv)


def test_deterministic():
    w = SMALL[-1]
    _say(f"determinism {w['name']}")
    inputs = make_workload_inputs(w)
    o1, l1 = run_gpu(*inputs)
    o2, l2 = run_gpu(*inputs)
    o3, l3 = run_gpu(*inputs)
    assert torch.equal(o1, o2) and torch.equal(o1, o3)
    assert torch.equal(l1, l2) and torch.equal(l1, l3)


def test_leak_probes():
    """Masks on the GPU: a changed key/value at position s leaves rows t < s
    bit-identical; a changed depth slot of position t' leaves rows t != t'
    bit-identical."""
    B, T, Hq, Hkv, d, L_d = 1, 300, 8, 2, 128, 6
    _say("leak probes")
    q, ks, vs, kd, vd = make_inputs(B, T, Hq, Hkv, d, L_d, dtype="bf16", seed=9)
    out, lse = run_gpu(q, ks, vs, kd, vd)
    for s in (0, 5, 64, 150, 299):
        ks2, vs2 = ks.clone(), vs.clone()
        ks2[:, s] = (ks2[:, s].float() + 1.5).to(ks.dtype)
        vs2[:, s] = (vs2[:, s].float() - 2.0).to(vs.dtype)
        out2, lse2 = run_gpu(q, ks2, vs2, kd, vd)
        assert torch.equal(out2[:, :s], out[:, :s]) and torch.equal(lse2[:, :, :s], lse[:, :, :s]), s
        assert not torch.equal(out2[:, s], out[:, s])
    for tp in (0, 31, 32, 299):
        kd2, vd2 = kd.clone(), vd.clone()
        kd2[:, tp] = (kd2[:, tp].float() + 1.5).to(kd.dtype)
        vd2[:, tp] = (vd2[:, tp].float() - 2.0).to(vd.dtype)
        out3, lse3 = run_gpu(q, ks, vs, kd2, vd2)
        others = [t for t in range(T) if t != tp]
        assert torch.equal(out3[:, others], out[:, others]) and torch.equal(lse3[:, :, others], lse[:, :, others]), tp
        assert not torch.equal(out3[:, tp], out[:, tp])


def test_without_lse_and_on_side_stream():
    B, T, Hq, Hkv, d, L_d = 1, 257, 8, 2, 128, 4
    _say("lse=None and a side stream")
    inputs = make_inputs(B, T, Hq, Hkv, d, L_d, dtype="bf16", seed=21)
    out_ref, _ = run_gpu(*inputs)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, lse = run_gpu(*inputs, with_lse=False, stream=s)
    assert lse is None
    assert torch.equal(out, out_ref)


def test_errors_raise():
    _say("error paths")
    q = torch.zeros(1, 4, 3, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moda.ModaError):
        moda.moda_fwd(q, k, k, None, None, 0)          # Hq % Hkv != 0
    q = torch.zeros(1, 4, 2, 96, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 1, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(moda.ModaError):
        moda.moda_fwd(q, k, k, None, None, 0)          # d = 96 not built
    q = torch.zeros(1, 4, 2, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):                    # caller's out too small
        moda.moda_fwd(q, k, k, None, None, 0, out=torch.empty(1, 2, 2, 128, dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):                    # caller's out of another dtype
        moda.moda_fwd(q, k, k, None, None, 0, out=torch.empty(1, 4, 2, 128, dtype=torch.float32, device="cuda"))


def test_counter_order_repeatable_and_concurrent():
    """Grids of several rounds take their query tiles from a per-launch
    counter slot that each launch returns to zero: calls in a row, and calls
    in flight at the same time on two streams, give bit-identical results
    (a slot left non-zero would make the next launch skip tiles), equal to
    the oracle on sampled rows."""
    B, T, Hq, Hkv, d, L = 1, 16384, 16, 2, 128, 4
    _say(f"counter order: B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} L_d={L} (8-wave grid, 4 rounds)")
    inputs = make_inputs(B, T, Hq, Hkv, d, L, dtype="bf16", seed=4242)
    dev = torch.device("cuda:0")
    q, ks, vs, kd, vd = [x.to(dev) for x in inputs]
    kp = torch.empty(moda.depth_packed_elems(B, T, Hkv, d, L), dtype=q.dtype, device=dev)
    vp = torch.empty_like(kp)
    moda.moda_pack_depth(kd, vd, kp, vp)
    outs = []
    for _ in range(3):
        o, l = moda.moda_fwd(q, ks, vs, kp, vp, L)
        outs.append((o, l))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    conc = []
    for _ in range(2):
        for s in (s1, s2):
            o = torch.empty_like(q)
            l = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                moda.moda_fwd(q, ks, vs, kp, vp, L, out=o, lse=l, stream=s)
            conc.append((o, l))
    torch.cuda.synchronize()
    o0, l0 = outs[0]
    for i, (o, l) in enumerate(outs[1:] + conc):
        assert torch.equal(o, o0) and torch.equal(l, l0), f"call {i + 1} differs from the first"
    rows = sample_rows(B, T, Hq, n=512, seed=4243, tile_rows=(T - 1,))
    _check("counter order", inputs[0].dtype, *compare_rows(inputs, o0.cpu(), l0.cpu(), rows))


def test_counter_order_under_graph_replay():
    """A forward and an allocation-free backward on long grids (tiles from the
    launch counters) recorded into a HIP graph: each replay, with eager work
    and synchronisations between replays, equals the eager results bit for
    bit (the recorded launches keep their counter slots, which each replay
    returns to zero)."""
    B, T, Hq, Hkv, d, L = 1, 16384, 16, 2, 128, 4
    _say(f"graph replay: B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} L_d={L}")
    from moda_inputs import make_dout
    dev = torch.device("cuda:0")
    q, ks, vs, kd, vd = [x.to(dev) for x in make_inputs(B, T, Hq, Hkv, d, L, dtype="bf16", seed=7171)]
    dout = make_dout(B, T, Hq, d, dtype="bf16", seed=7172).to(dev)
    kp, vp = moda.moda_pack_depth(kd, vd)
    ref_o, ref_l = moda.moda_fwd(q, ks, vs, kp, vp, L)
    ref_g = moda.moda_bwd(q, ks, vs, kp, vp, L, ref_o, ref_l, dout)
    o = torch.empty_like(ref_o)
    l = torch.empty_like(ref_l)
    g = tuple(torch.empty_like(x) for x in ref_g)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on the capture stream
        moda.moda_fwd(q, ks, vs, kp, vp, L, out=o, lse=l)
        moda.moda_bwd_noalloc(q, ks, vs, kp, vp, L, o, l, dout, grads=g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moda.moda_fwd(q, ks, vs, kp, vp, L, out=o, lse=l)
        moda.moda_bwd_noalloc(q, ks, vs, kp, vp, L, o, l, dout, grads=g)
    for r in range(3):
        o.zero_()
        for x in g:
            x.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), f"replay {r}: forward differs"
        for name, a, b in zip(("dq", "dk_seq", "dv_seq", "dk_depth", "dv_depth"), ref_g, g):
            assert torch.equal(a, b), f"replay {r}: {name} differs"
        # eager work between replays, on the same counters' ring
        moda.moda_fwd(q, ks, vs, kp, vp, L)
        torch.cuda.synchronize()


def test_ragged_long_grid_sampled_rows():
    """A long grid (tiles from the launch counter) whose length is not a
    multiple of the 64-key block or of the 32-key depth tile: T = 20001,
    G = 8, L_d = 5.  Sampled rows (with the last positions, where the last
    key block and the last depth tile are partial) against the oracle."""
    B, T, Hq, Hkv, d, L = 1, 20001, 16, 2, 128, 5
    _say(f"ragged long grid: B={B} T={T} Hq={Hq} Hkv={Hkv} d={d} L_d={L}")
    inputs = make_inputs(B, T, Hq, Hkv, d, L, dtype="bf16", seed=8181)
    rows = sample_rows(B, T, Hq, n=1024, seed=8182, tile_rows=(T - 1, T - 2, T - 33, 19968, 19967))
    out, lse = run_gpu(*inputs)
    _check("ragged long grid", inputs[0].dtype, *compare_rows(inputs, out, lse, rows))
