"""Benchmark of the MoDA forward hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the depth repack (moda_pack_depth) followed by the fused forward (moda_fwd).
Inputs are resident in HBM before the timed region starts.

Prints ONE JSON line (rank 0, one GPU):
  value        useful TFLOP/s of the step (pack + fwd),
               useful FLOPs = 4 * B * Hq * d * (T (T+1) / 2 + T * L_d)
  roofline     the fused forward kernel against the bf16 dense matrix-core
               peak, from HIP events around each launch in the timed region
  cpu_baseline the oracle timed on the host on a bounded sample of rows
plus the forward-only rate, the repack time and bandwidth, and the forward
time of the same kernel at L_d = 0 (overhead of the depth slots).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoDA fwd TFLOP/s (bf16, T=64K) + % MFMA peak; overhead vs L_d=0"
DEFAULT_WORKLOAD = "bf16_B1_T65536_Hq16_Hkv2_d128_L24"
PEAK_TFLOPS = {"bf16": 2500.0, "fp32": 157.3}   # MI355X dense matrix-core peaks
HBM_PEAK_GBPS = 8000.0
FLUSH_BYTES = 512 << 20                             # > L2 + the 256 MB MALL
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def useful_flops(B, T, Hq, d, L_d, rows=None):
    """QK^T and PV multiply-adds of unmasked scores, 2 flops each."""
    if rows is None:
        return 4.0 * B * Hq * d * (T * (T + 1) / 2 + T * L_d)
    return float(sum(4.0 * d * (int(t) + 1 + L_d) for (_, t, _) in rows))


def compulsory_bytes(w):
    eb = 2 if w["dtype"] == "bf16" else 4
    B, T, Hq, Hkv, d, L = w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"]
    return eb * (2 * B * T * Hq * d + 2 * B * T * Hkv * d + 2 * B * T * L * Hkv * d) + 4 * B * Hq * T


FWD_SOURCES = ("moda_common.hpp", "moda_fwd.hpp", "moda_fwd_bf16.hpp")


def _code_only(text):
    """C++ source without its comments and blank space, so that an edit of a
    comment does not count as a change of the kernel."""
    out, i, n = [], 0, len(text)
    while i < n:
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif text[i] == '"':                      # string literal, kept whole
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(text[i])
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash():
    """Hash of the code (comments and spacing aside) of the sources the fused
    forward kernel is compiled from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "depth_augmented_attention_amd", "csrc")
    for f in FWD_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per fused-forward launch from the committed rocprofv3 counter
    summary of this workload, if it was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"moda_fwd_{workload}_hbm_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def cpu_baseline(w, inputs, budget_s, out_cpu=None, lse_cpu=None):
    """Oracle rate on a bounded, seeded sample of query rows of the workload.

    When the timed forward's out / lse (CPU copies) are given, the sampled
    rows are also compared with them: max |out - oracle| and max |lse - oracle|
    over those rows."""
    import numpy as np
    import torch

    from moda_inputs import sample_rows
    from oracle import moda_forward
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas = None
    cores = len(os.sched_getaffinity(0))
    q, ks, vs, kd, vd = [x.to(torch.float32).numpy() for x in inputs]
    B, T, Hq, L_d = w["B"], w["T"], w["Hq"], w["L_d"]
    rows = sample_rows(B, T, Hq, n=65536, seed=w["seed"] + 11)
    rng = np.random.default_rng(w["seed"] + 12)
    rows = rows[rng.permutation(len(rows))]
    done = 0
    flops = 0.0
    err_o = err_l = 0.0
    c0 = time.process_time()
    t0 = time.perf_counter()
    chunk = 64
    while done < len(rows) and time.perf_counter() - t0 < budget_s:
        sel = rows[done:done + chunk]
        ro, rl = moda_forward(q, ks, vs, kd, vd, rows=sel)
        if out_cpu is not None:
            b_, t_, h_ = sel[:, 0], sel[:, 1], sel[:, 2]
            err_o = max(err_o, float(np.abs(out_cpu[b_, t_, h_].astype(np.float64) - ro).max()))
            err_l = max(err_l, float(np.abs(lse_cpu[b_, h_, t_].astype(np.float64) - rl).max()))
        flops += useful_flops(B, T, Hq, w["d"], L_d, rows=sel)
        done += len(sel)
    dt = time.perf_counter() - t0
    busy = (time.process_time() - c0) / dt      # CPU seconds per wall second, all threads
    # the oracle's cost of a row is proportional to its key count t + 1 + L_d
    keys_done = float(sum(int(t) + 1 + L_d for t in rows[:done, 1]))
    keys_all = float(B * Hq) * (T * (T + 1) / 2 + T * L_d)
    res = {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} seeded random (b,t,h) query rows of {w['name']} "
                  f"(float64 numpy oracle, {dt:.1f} s; rate = useful FLOPs of those rows / time)",
        "cpu_model": cpu_model(),
        "blas_threads": blas,
        "rows_per_s": done / dt,
        "cpu_seconds_per_wall_second": busy,
        "projected_full_output_s": dt * keys_all / keys_done,
        "projection": "measured time x (keys of all rows) / (keys of the sampled rows): a projection, not a run",
    }
    if out_cpu is not None:
        res["max_abs_err_out"] = err_o
        res["max_abs_err_lse"] = err_l
        res["err_rows"] = done
    return res


def gpu_clock_under_load(launch, seconds=2.5):
    """sclk (MHz) that rocm-smi reports while `launch` keeps the GPU busy
    (enough launches queued for about `seconds`), and the highest sclk level."""
    import subprocess

    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    launch()
    ev[1].record()
    torch.cuda.synchronize()
    n = max(1, int(seconds * 1e3 / max(ev[0].elapsed_time(ev[1]), 1e-3)))
    for _ in range(n):
        launch()
    time.sleep(0.4)
    cur = top = None
    try:
        import re
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        for line in r.stdout.splitlines():
            m = re.search(r"(\d+)\s*Mhz", line)
            if "sclk" in line and m:
                cur = float(m.group(1))
                break
        r = subprocess.run(["rocm-smi", "--showclkfrq"], capture_output=True, text=True, timeout=20)
        sec = False
        for line in r.stdout.splitlines():
            if "frequencies" in line:
                sec = "sclk" in line.lower()
                continue
            m = re.search(r"(\d+)\s*Mhz", line)
            if sec and m:
                top = max(top or 0.0, float(m.group(1)))
    except Exception:  # pragma: no cover
        pass
    torch.cuda.synchronize()
    return cur, top


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-l0", action="store_true", help="skip the L_d = 0 comparison")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the write-step and depth-window measurements")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward measurement")
    ap.add_argument("--bwd-ws", action="store_true",
                    help="time the backward through moda_bwd_ws (row-split dK/dV on short sequences)")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the depth-overhead sweep over the other bf16 workloads")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the fused kernel's sharding across GPUs is described in the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import depth_augmented_attention_amd as moda
    from moda_inputs import make_workload_inputs, workload

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 1 GiB")
        return

    w = workload(args.workload)
    B, T, Hq, Hkv, d, L_d = w["B"], w["T"], w["Hq"], w["Hkv"], w["d"], w["L_d"]
    log(f"workload {w['name']}: generating seeded inputs")
    inputs = make_workload_inputs(w)
    q, ks, vs, kd, vd = [x.to(dev) for x in inputs]
    kp = torch.empty(moda.depth_packed_elems(B, T, Hkv, d, L_d), dtype=q.dtype, device=dev)
    vp = torch.empty_like(kp)
    out = torch.empty_like(q)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        moda.moda_pack_depth(kd, vd, kp, vp)
        if ev is not None:
            ev[1].record()
        moda.moda_fwd(q, ks, vs, kp, vp, L_d, out=out, lse=lse)
        if ev is not None:
            ev[2].record()

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    log(f"timing {args.steps} steps")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    pack_ms = [e[0].elapsed_time(e[1]) for e in evs]
    fwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    ms_per_step = wall * 1e3 / args.steps
    avg_fwd = sum(fwd_ms) / len(fwd_ms)
    avg_pack = sum(pack_ms) / len(pack_ms)
    med = lambda xs: sorted(xs)[len(xs) // 2]
    # the timed forward's results, compared with the oracle's sampled rows below
    out_cpu = out.to(torch.float32).cpu().numpy() if not args.no_cpu_baseline else None
    lse_cpu = lse.cpu().numpy() if not args.no_cpu_baseline else None
    F = useful_flops(B, T, Hq, d, L_d)
    log(f"step {ms_per_step:.3f} ms  fwd {avg_fwd:.3f} ms  pack {avg_pack:.3f} ms")

    res = {
        "metric": METRIC,
        "value": F / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w["dtype"],
        "data": "synthetic (seeded i.i.d. N(0,1), rounded to bf16)",
        "config": {"workload": w["name"], "B": B, "T": T, "Hq": Hq, "Hkv": Hkv, "d": d, "L_d": L_d,
                   "step": "moda_pack_depth + moda_fwd"},
    }
    fwd_tflops = F / (avg_fwd * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w["dtype"]]
    traffic = measured_traffic(w["name"])
    res["roofline"] = {
        "bound": "mfma",
        "kernel": "moda_fwd_bf16_kernel" if w["dtype"] == "bf16" else "moda_fwd_kernel",
        "achieved": fwd_tflops,
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": fwd_tflops / peak,
        "traffic": traffic,
        "avg_launch_ms": avg_fwd,
    }
    res["fwd_ms"] = avg_fwd
    res["fwd_ms_median"] = med(fwd_ms)
    res["step_ms_median"] = med([a + b for a, b in zip(pack_ms, fwd_ms)])
    res["fwd_tflops"] = fwd_tflops
    res["fwd_tflops_median"] = F / (med(fwd_ms) * 1e-3) / 1e12
    res["pct_mfma_peak"] = 100.0 * fwd_tflops / peak
    res["pack_ms"] = avg_pack
    res["pack_gbps"] = 2 * 2 * kd.numel() * kd.element_size() / (avg_pack * 1e-3) / 1e9
    res["fwd_compulsory_gbps"] = compulsory_bytes(w) / (avg_fwd * 1e-3) / 1e9

    # Cache flush: a 512 MiB fill before each launch timed on its own, so that
    # neither L2 nor the 256 MB MALL still holds that launch's inputs (in the
    # timed steps above the depth repack, which streams 3.2 GB, does this).
    flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    res["cache_flush_bytes"] = FLUSH_BYTES

    def timed_launches(fns, reps):
        """Per-launch times (ms) of each function in fns, the functions taken
        in turn (so that both see the same clock and temperature), each launch
        after a cache flush; HIP events on the current stream around the
        launch only."""
        ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
              for _ in fns]
        for i in range(reps):
            for f, fn in enumerate(fns):
                flush_buf.fill_(i & 0xFF)
                ev[f][i][0].record()
                fn()
                ev[f][i][1].record()
        torch.cuda.synchronize()
        return [[a.elapsed_time(b) for a, b in e] for e in ev]

    if not args.no_l0 and L_d > 0:
        log("timing the same kernel at L_d = 0")
        for _ in range(2):
            moda.moda_fwd(q, ks, vs, None, None, 0, out=out, lse=lse)
        torch.cuda.synchronize()
        # the same kernel with and without the depth slots, alternating, each
        # launch after the cache fill
        ld, l0 = timed_launches([lambda: moda.moda_fwd(q, ks, vs, kp, vp, L_d, out=out, lse=lse),
                                 lambda: moda.moda_fwd(q, ks, vs, None, None, 0, out=out, lse=lse)], args.steps)
        avg_l0 = sum(l0) / len(l0)
        avg_ld = sum(ld) / len(ld)
        res["fwd_ms_L0"] = avg_l0
        res["fwd_ms_flushed"] = avg_ld
        res["fwd_ms_L0_median"] = med(l0)
        res["fwd_ms_flushed_median"] = med(ld)
        res["overhead_vs_L0_median"] = med(ld) / med(l0) - 1.0
        res["fwd_tflops_L0"] = useful_flops(B, T, Hq, d, 0) / (avg_l0 * 1e-3) / 1e12
        res["overhead_vs_L0"] = avg_ld / avg_l0 - 1.0
        res["overhead_vs_L0_with_pack"] = (avg_ld + avg_pack) / avg_l0 - 1.0
        # depth stream: its bytes over the time the depth slots add to the
        # forward (above the HBM peak means the stream is hidden under the sweep)
        depth_stream_bytes = 2.0 * B * T * L_d * Hkv * d * q.element_size()
        res["depth_stream_bytes"] = depth_stream_bytes
        res["depth_incremental_ms"] = avg_ld - avg_l0
        res["depth_stream_gbps_incremental"] = (depth_stream_bytes / ((avg_ld - avg_l0) * 1e-3) / 1e9
                                                if avg_ld > avg_l0 else None)
        log(f"L_d=0 fwd {avg_l0:.3f} ms, overhead {100 * res['overhead_vs_L0']:.2f}%")

    if not args.no_extras and L_d > 0:
        # write step: this layer's K/V appended as one slot of the packed buffers
        log("timing the write step (one slot append) and a depth window")
        reps = 10
        ea = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        moda.moda_append_depth(ks, vs, kp, vp, L_d, L_d - 1)
        torch.cuda.synchronize()
        ea[0].record()
        for i in range(reps):
            moda.moda_append_depth(ks, vs, kp, vp, L_d, L_d - 1)
            ea[i + 1].record()
        torch.cuda.synchronize()
        app_ms = sum(ea[i].elapsed_time(ea[i + 1]) for i in range(reps)) / reps
        app_bytes = 2 * 2 * ks.numel() * ks.element_size()
        res["append_ms"] = app_ms
        res["append_gbps"] = app_bytes / (app_ms * 1e-3) / 1e9
        res["append_hbm_frac"] = res["append_gbps"] / HBM_PEAK_GBPS
        # bounded window: the last 8 of the L_d slots
        lo = max(0, L_d - 8)
        ew = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        moda.moda_fwd_window(q, ks, vs, kp, vp, L_d, lo, L_d, out=out, lse=lse)
        torch.cuda.synchronize()
        ew[0].record()
        for i in range(3):
            moda.moda_fwd_window(q, ks, vs, kp, vp, L_d, lo, L_d, out=out, lse=lse)
            ew[i + 1].record()
        torch.cuda.synchronize()
        win_ms = sum(ew[i].elapsed_time(ew[i + 1]) for i in range(3)) / 3
        res["window_slots"] = [lo, L_d]
        res["window_fwd_ms"] = win_ms
        res["window_fwd_tflops"] = (4.0 * B * Hq * d * (T * (T + 1) / 2 + T * (L_d - lo))) / (win_ms * 1e-3) / 1e12
        if "fwd_ms_L0" in res:
            res["window_overhead_vs_L0"] = win_ms / res["fwd_ms_L0"] - 1.0
        # 8-bit depth KV: quantising repack and the forward over int8 codes
        log("timing 8-bit depth KV (pack_q8, fwd_q8)")
        packed = moda.moda_pack_depth_q8(kd, vd)
        moda.moda_fwd_q8(q, ks, vs, packed, L_d, out=out, lse=lse)
        torch.cuda.synchronize()
        # repack into the same buffers: median of 10 calls, each timed alone
        ep = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
        for a_, b_ in ep:
            a_.record()
            moda.moda_pack_depth_q8(kd, vd, out=packed)
            b_.record()
        eq = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        eq[0].record()
        for i in range(3):
            moda.moda_fwd_q8(q, ks, vs, packed, L_d, out=out, lse=lse)
            eq[1 + i].record()
        torch.cuda.synchronize()
        q8_pack_ms = med([a_.elapsed_time(b_) for a_, b_ in ep])
        q8_fwd_ms = eq[0].elapsed_time(eq[3]) / 3
        depth_elems = kd.numel()
        q8_bytes = 2 * depth_elems + 2 * 4 * (depth_elems // d)       # codes + row scales, K and V
        res["q8_depth_bytes"] = q8_bytes
        res["depth_bytes"] = 2 * depth_elems * kd.element_size()
        res["q8_pack_ms"] = q8_pack_ms
        res["q8_pack_gbps"] = (res["depth_bytes"] + q8_bytes) / (q8_pack_ms * 1e-3) / 1e9
        res["q8_fwd_ms"] = q8_fwd_ms
        res["q8_fwd_tflops"] = F / (q8_fwd_ms * 1e-3) / 1e12
        if "fwd_ms_L0" in res:
            res["q8_overhead_vs_L0"] = q8_fwd_ms / res["fwd_ms_L0"] - 1.0
        if not args.no_bwd:
            # backward over the 8-bit depth KV (mean of 2 calls after one warm-up)
            from moda_inputs import make_dout
            dq8 = make_dout(B, T, Hq, d, dtype=w["dtype"], seed=w["seed"]).to(q.device)
            moda.moda_fwd_q8(q, ks, vs, packed, L_d, out=out, lse=lse)
            g8 = moda.moda_bwd_q8(q, ks, vs, packed, L_d, out, lse, dq8)
            torch.cuda.synchronize()
            e8 = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e8[0].record()
            for i in range(2):
                moda.moda_bwd_q8(q, ks, vs, packed, L_d, out, lse, dq8, grads=g8)
                e8[i + 1].record()
            torch.cuda.synchronize()
            res["q8_bwd_ms"] = e8[0].elapsed_time(e8[2]) / 2
            del g8, dq8
        del packed

    if not args.no_sweep:
        # overhead of the depth slots on the other bf16 workloads (G and depth
        # sweep): forward with depth vs the same kernel at L_d = 0, inputs N(0,1)
        # drawn on the GPU (timing only)
        from moda_inputs import WORKLOADS
        sweep = {}
        for ws in WORKLOADS:
            if ws["dtype"] != "bf16" or ws["name"] == w["name"]:
                continue
            log(f"sweep {ws['name']}")
            sB, sT, sHq, sHkv, sd, sL = ws["B"], ws["T"], ws["Hq"], ws["Hkv"], ws["d"], ws["L_d"]
            g = torch.Generator(device=dev).manual_seed(ws["seed"])
            rn = lambda *sh: torch.randn(*sh, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
            sq, sk, sv = rn(sB, sT, sHq, sd), rn(sB, sT, sHkv, sd), rn(sB, sT, sHkv, sd)
            skd, svd = rn(sB, sT, sL, sHkv, sd), rn(sB, sT, sL, sHkv, sd)
            skp, svp = moda.moda_pack_depth(skd, svd)
            so = torch.empty_like(sq)
            sl = torch.empty(sB, sHq, sT, dtype=torch.float32, device=dev)
            reps = 20 if sT <= 16384 else 5

            moda.moda_fwd(sq, sk, sv, skp, svp, sL, out=so, lse=sl)
            moda.moda_fwd(sq, sk, sv, None, None, 0, out=so, lse=sl)
            torch.cuda.synchronize()
            td, t0 = timed_launches([lambda: moda.moda_fwd(sq, sk, sv, skp, svp, sL, out=so, lse=sl),
                                     lambda: moda.moda_fwd(sq, sk, sv, None, None, 0, out=so, lse=sl)], reps)
            t_d = sorted(td)[reps // 2]                        # medians, each launch after a cache flush
            t_0 = sorted(t0)[reps // 2]
            Fs = useful_flops(sB, sT, sHq, sd, sL)
            sweep[ws["name"]] = {"fwd_ms": t_d, "fwd_ms_L0": t_0, "overhead_vs_L0": t_d / t_0 - 1.0,
                                 "fwd_tflops": Fs / (t_d * 1e-3) / 1e12, "reps": reps}
            if moda.fwd_workspace_bytes(sB, sT, sHq, sHkv, sd, sq.dtype) > 0:
                # the same workload through moda_fwd_ws (longest tiles' key
                # ranges split over two workgroups)
                wk = moda.fwd_workspace(sq, sk)
                moda.moda_fwd(sq, sk, sv, skp, svp, sL, out=so, lse=sl, work=wk)
                torch.cuda.synchronize()
                tw, tw0 = timed_launches(
                    [lambda: moda.moda_fwd(sq, sk, sv, skp, svp, sL, out=so, lse=sl, work=wk),
                     lambda: moda.moda_fwd(sq, sk, sv, None, None, 0, out=so, lse=sl, work=wk)], reps)
                t_w, t_w0 = sorted(tw)[reps // 2], sorted(tw0)[reps // 2]
                sweep[ws["name"]].update({"ws_fwd_ms": t_w, "ws_fwd_ms_L0": t_w0,
                                          "ws_fwd_tflops": Fs / (t_w * 1e-3) / 1e12,
                                          "ws_overhead_vs_L0": t_w / t_w0 - 1.0})
                del wk
            if not args.no_bwd and sT <= 16384:
                # the backward of this workload: moda_bwd, and moda_bwd_ws
                # where it splits the dK/dV rows (short sequences)
                sdo = rn(sB, sT, sHq, sd)
                moda.moda_fwd(sq, sk, sv, skp, svp, sL, out=so, lse=sl)
                sg = moda.moda_bwd(sq, sk, sv, skp, svp, sL, so, sl, sdo)
                swk = torch.empty(2, sB, sHq, sT, dtype=torch.float32, device=dev)
                fns = [lambda: moda.moda_bwd(sq, sk, sv, skp, svp, sL, so, sl, sdo, grads=sg, work=swk)]
                split = moda.bwd_workspace_bytes(sB, sT, sHq, sHkv, sd, sq.dtype) > swk.numel() * 4 + 255
                if split:
                    bws = moda.bwd_workspace(sq, sk)
                    fns.append(lambda: moda.moda_bwd(sq, sk, sv, skp, svp, sL, so, sl, sdo, grads=sg, workspace=bws))
                for f in fns:
                    f()
                torch.cuda.synchronize()
                tb = timed_launches(fns, 5)
                sweep[ws["name"]]["bwd_ms"] = med(tb[0])
                sweep[ws["name"]]["bwd_tflops"] = 2.5 * Fs / (med(tb[0]) * 1e-3) / 1e12
                if split:
                    sweep[ws["name"]]["ws_bwd_ms"] = med(tb[1])
                    sweep[ws["name"]]["ws_bwd_tflops"] = 2.5 * Fs / (med(tb[1]) * 1e-3) / 1e12
                    del bws
                del sdo, sg, swk
            del sq, sk, sv, skd, svd, skp, svp, so, sl
        res["overhead_sweep"] = sweep

    if not args.no_sweep and w["dtype"] == "bf16":
        # depth sweep at the bench shape: the same kernel with L_d = 0, 12, 24
        # and 48 slots (inputs N(0,1) drawn on the GPU: timing only), launches
        # of the four taken in turn, each after the cache fill; medians
        log("depth sweep L_d = 0, 12, 24, 48")
        g = torch.Generator(device=dev).manual_seed(w["seed"] + 99)
        Lmax = 48
        kdx = torch.randn(B, T, Lmax, Hkv, d, generator=g, device=dev, dtype=torch.float32).to(q.dtype)
        vdx = torch.randn(B, T, Lmax, Hkv, d, generator=g, device=dev, dtype=torch.float32).to(q.dtype)
        packs = {}
        for Lx in (12, 24, 48):
            packs[Lx] = moda.moda_pack_depth(kdx[:, :, :Lx].contiguous(), vdx[:, :, :Lx].contiguous())
        del kdx, vdx
        fns = [lambda: moda.moda_fwd(q, ks, vs, None, None, 0, out=out, lse=lse)]
        for Lx in (12, 24, 48):
            fns.append(lambda Lx=Lx: moda.moda_fwd(q, ks, vs, packs[Lx][0], packs[Lx][1], Lx, out=out, lse=lse))
        for f in fns:
            f()
        torch.cuda.synchronize()
        times = timed_launches(fns, 5)
        t0m = med(times[0])
        dsw = {"L_d": [0, 12, 24, 48], "fwd_ms_median": [med(t) for t in times],
               "overhead_vs_L0": [med(t) / t0m - 1.0 for t in times]}
        # least-squares line through the added time: linear in L_d if the
        # residuals are small against the slope
        xs = [0.0, 12.0, 24.0, 48.0]
        ys = [med(t) - t0m for t in times]
        xm, ym = sum(xs) / 4, sum(ys) / 4
        slope = sum((x - xm) * (y - ym) for x, y in zip(xs, ys)) / sum((x - xm) ** 2 for x in xs)
        dsw["added_ms_per_slot"] = slope
        dsw["fit_residual_ms_max"] = max(abs(y - (ym + slope * (x - xm))) for x, y in zip(xs, ys))
        res["depth_sweep"] = dsw
        del packs
        log("depth sweep: " + ", ".join(f"L{x} {y:.3f} ms" for x, y in zip(dsw["L_d"], dsw["fwd_ms_median"])))
        # the clock the forward runs at: rocm-smi's sclk while the forward
        # keeps the GPU busy
        cur, top = gpu_clock_under_load(lambda: moda.moda_fwd(q, ks, vs, kp, vp, L_d, out=out, lse=lse))
        res["gpu_sclk_mhz_under_load"] = cur
        res["gpu_sclk_mhz_max"] = top
        log(f"sclk under load {cur} MHz (max {top} MHz)")
        # context for the pages' comparison with FlashAttention-2 (their
        # kernel at 97.3% of its efficiency at 64K): PyTorch's own
        # flash-attention backend on the same GPU, plain causal attention at
        # this shape (K/V heads repeated to Hq), launches after the cache fill
        # taken in turn with moda_fwd at L_d = 0; the flash backend only (no
        # fallback to another backend)
        try:
            from torch.nn.attention import SDPBackend, sdpa_kernel
            qt = q.transpose(1, 2).contiguous()
            kt = ks.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1).contiguous()
            vt = vs.transpose(1, 2).repeat_interleave(Hq // Hkv, dim=1).contiguous()

            def sdpa():
                with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                    return torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True)
            sdpa()
            moda.moda_fwd(q, ks, vs, None, None, 0, out=out, lse=lse)
            torch.cuda.synchronize()
            ts, tm = timed_launches([sdpa, lambda: moda.moda_fwd(q, ks, vs, None, None, 0, out=out, lse=lse)], 5)
            F0 = useful_flops(B, T, Hq, d, 0)
            sd = {"backend": "torch SDPA, FLASH_ATTENTION", "ms_median": med(ts),
                  "tflops": F0 / (med(ts) * 1e-3) / 1e12, "moda_fwd_L0_ms_median": med(tm),
                  "moda_fwd_L0_tflops": F0 / (med(tm) * 1e-3) / 1e12}
            # useful TFLOP/s of the timed MoDA forward (with its depth slots)
            # over the library's plain causal attention
            sd["moda_vs_sdpa_efficiency"] = res["fwd_tflops"] / sd["tflops"]
            res["torch_sdpa_flash_L0"] = sd
            del qt, kt, vt
            log(f"torch SDPA flash (L_d = 0): {sd['ms_median']:.3f} ms, {sd['tflops']:.1f} TFLOP/s")
        except Exception as e:      # backend missing on this build: recorded, not fatal
            res["torch_sdpa_flash_L0"] = {"unavailable": f"{type(e).__name__}: {str(e)[:200]}"}

    if not args.no_bwd:
        # backward of the same forward: dq, dk/dv of sequence and depth keys
        from moda_inputs import make_dout
        log("timing the backward (" + ("moda_bwd_ws" if args.bwd_ws else "moda_bwd") + ")")
        moda.moda_fwd(q, ks, vs, kp, vp, L_d, out=out, lse=lse)
        dout = make_dout(B, T, Hq, d, dtype=w["dtype"], seed=w["seed"]).to(q.device)
        bws = moda.bwd_workspace(q, ks) if args.bwd_ws else None
        grads = moda.moda_bwd(q, ks, vs, kp, vp, L_d, out, lse, dout, workspace=bws)
        torch.cuda.synchronize()
        reps = 3
        eb = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        eb[0].record()
        for i in range(reps):
            moda.moda_bwd(q, ks, vs, kp, vp, L_d, out, lse, dout, grads=grads, workspace=bws)
            eb[i + 1].record()
        torch.cuda.synchronize()
        bwd_ms = sum(eb[i].elapsed_time(eb[i + 1]) for i in range(reps)) / reps
        # useful work: five products over the unmasked scores (S recomputed,
        # dP, dV, dQ, dK), 2.5x the forward's two; the kernels execute seven
        # (S and dP are formed once for dq and once for dk/dv)
        res["bwd_ms"] = bwd_ms
        res["bwd_entry"] = "moda_bwd_ws" if args.bwd_ws else "moda_bwd"
        res["bwd_tflops"] = 2.5 * F / (bwd_ms * 1e-3) / 1e12
        res["bwd_frac_mfma_peak"] = res["bwd_tflops"] / peak
        log(f"bwd {bwd_ms:.3f} ms  {res['bwd_tflops']:.1f} TFLOP/s")
        del grads, dout, bws

    if not args.no_cpu_baseline:
        log(f"oracle on host cores ({args.cpu_budget:.0f} s budget)")
        del q, ks, vs, kd, vd
        res["cpu_baseline"] = cpu_baseline(w, inputs, args.cpu_budget, out_cpu, lse_cpu)
        res["max_abs_err_out"] = res["cpu_baseline"].get("max_abs_err_out")
        res["max_abs_err_lse"] = res["cpu_baseline"].get("max_abs_err_lse")
    else:
        res["cpu_baseline"] = None
    res["kernel_source_hash"] = kernel_source_hash()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
