#!/usr/bin/env python3
"""Headline benchmark: activation-sparse GEMV at 50% sparsity on the
Llama-2-7B down projection (W 4096 x 11008 fp16, batch 1).

One step = one pass of the hot path over one synthetic activation: magnitude
threshold (calibrated for 50% sparsity from 10k synthetic samples by the
library's own calibration kernel) and the sparse GEMV over the surviving
weight columns -- one fused launch, ``sparse_gemv_threshold``.  The weight
rotates through distinct copies totalling >= 1 GiB so every step streams its
kept columns from HBM rather than from the 256 MB Infinity Cache.

Prints one JSON line (rank 0).  ``value`` is microseconds per step (lower is
better): the median of ten windows of --steps back-to-back steps each, every
window between two HIP events on the launch stream (``windows`` gives the
minimum and maximum).  The roofline object gives the effective HBM bandwidth
on the bytes the method must touch, against the 8 TB/s MI355X peak.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("sparse GEMV µs + effective HBM GB/s (% of peak) at 50% sparsity, "
          "4096×11008 fp16")
HBM_PEAK_GBS = 8000.0
D_OUT, D_IN = 4096, 11008
SPARSITY = 0.5
ROTATION_BYTES = 1 << 30
COPY_BYTES = 256 << 20
GEMV_SOURCE = os.path.join(ROOT, "sparse_input_gemv_amd", "csrc", "gemv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_sparse_gemv_threshold_down_4096x11008.json")
NUM_WINDOWS = 10  # timed windows of --steps steps each; the headline is their median


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--graph", action="store_true", help="replay the steps from a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=16.0)
    ap.add_argument("--tiling", type=int, default=-1, help="GEMV tiling override (tuning)")
    ap.add_argument("--target-wgs", type=int, default=0, help="GEMV workgroup target (tuning)")
    ap.add_argument("--handoff", type=int, default=0, choices=[0, 1, 2, 3],
                    help="split-K partial sum: 0 auto, 1 second launch, 2 same launch, 3 same launch in L2 (tuning)")
    ap.add_argument("--only", choices=["fused", "unfused", "dense", "read"], default=None,
                    help="time a single path (for profiler runs)")
    ap.add_argument("--rows", default=None,
                    help="with --suite: comma-separated rows to run (read, config1, a1..a9, "
                         "next1..next4); "
                         "default all")
    ap.add_argument("--suite", action="store_true",
                    help="instead of the headline line, time every hot-path row on its "
                         "workload and print one JSON line per measurement")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy 5 times, so hardware byte "
                         "counters can be scaled against a kernel of known traffic")
    return ap.parse_args()


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(bytes_per_launch_hint: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None.

    The file records the hash of the GEMV source it was measured on; once
    the kernel changes the counters no longer apply and None is returned.
    """
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    if tr.get("gemv_source_sha256_16") != source_hash(GEMV_SOURCE):
        return None
    return tr.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sparse GEMV would shard by d_out with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_input_gemv_amd as sa
    import synthetic as syn

    if args.suite:
        run_suite(args)
        return

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = sa.lib()
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream

    # ---- inputs -------------------------------------------------------------
    wt0 = torch.from_numpy(syn.weight_t(D_OUT, D_IN, syn.weight_seed("down"))).to(dev)
    copies = max(2, -(-ROTATION_BYTES // wt0.numel() // 2))
    rot = [wt0] + [torch.roll(wt0, shifts=997 * i, dims=0).contiguous() for i in range(1, copies)]
    x_np = syn.activation((D_IN,), "laplace", 0)
    x = torch.from_numpy(x_np).to(dev)
    samples = torch.from_numpy(syn.calibration_samples("down_in")).to(dev)
    t = float(sa.act_calibrate_threshold(samples, SPARSITY).cpu()[0])
    mask, idx, val, nnz_t = sa.act_sparsify_threshold(x, t)
    nnz = int(nnz_t.cpu()[0])
    y = torch.empty((D_OUT,), dtype=torch.float16, device=dev)
    ws_bytes = sa.workspace_bytes(D_OUT, D_IN, 1)
    ws = sa.workspace(dev, ws_bytes)
    if args.tiling >= 0 or args.target_wgs > 0 or args.handoff > 0:
        sa.set_gemv_tuning(args.tiling, args.target_wgs, args.handoff)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 2, dtype=torch.float16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    # prebuilt C-ABI argument lists: the timed loop does no Python-side work
    # beyond the ctypes call
    fused = [(L.sparse_gemv_threshold,
              (w.data_ptr(), D_OUT, D_IN, x.data_ptr(), 1, t, y.data_ptr(), ws.data_ptr(),
               ws.numel(), sptr)) for w in rot]
    sparsify = (L.act_sparsify_threshold,
                (x.data_ptr(), 1, D_IN, t, mask.data_ptr(), idx.data_ptr(), val.data_ptr(),
                 nnz_t.data_ptr(), D_IN, sptr))
    listed = [(L.sparse_gemv,
               (w.data_ptr(), D_OUT, D_IN, idx.data_ptr(), val.data_ptr(), nnz_t.data_ptr(), 1,
                D_IN, y.data_ptr(), ws.data_ptr(), ws.numel(), sptr)) for w in rot]
    dense = [(L.dense_gemv,
              (w.data_ptr(), D_OUT, D_IN, x.data_ptr(), 1, y.data_ptr(), ws.data_ptr(),
               ws.numel(), sptr)) for w in rot]
    # achievable read rate: a plain contiguous read of the headline's
    # algorithmic bytes from the same rotation
    read_bytes = (2 * D_OUT * nnz + 2 * D_IN + 2 * D_OUT) // 16 * 16
    sink = torch.empty(sa.READ_STREAM_SINK_WORDS, dtype=torch.int32, device=dev)
    readp = [(L.sa_read_stream, (w.data_ptr(), read_bytes, sink.data_ptr(), sptr)) for w in rot]

    # cycles of torch's GPU sleep per millisecond, measured once
    torch.cuda._sleep(1000)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    torch.cuda._sleep(2_000_000)
    e1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = 2_000_000 / max(e0.elapsed_time(e1), 1e-3)

    def hold(ms):
        torch.cuda._sleep(int(cycles_per_ms * ms))

    def run(calls_per_step, steps, start=0):
        n = len(calls_per_step)
        for i in range(start, start + steps):
            for f, a in calls_per_step[i % n]:
                st = f(*a)
                if st != 0:
                    raise RuntimeError(L.sa_last_error().decode())

    def timed(calls_per_step, steps, warmup):
        """ms per step in each of NUM_WINDOWS windows of `steps` steps (one
        window of replays with --graph)."""
        run(calls_per_step, warmup)
        torch.cuda.synchronize()
        if args.graph:
            g = torch.cuda.CUDAGraph()
            per = len(calls_per_step)
            with torch.cuda.graph(g):
                cap_stream = torch.cuda.current_stream().cuda_stream
                for f, a in [c for step in calls_per_step for c in step]:
                    a = list(a)
                    a[-1] = cap_stream
                    if f(*a) != 0:
                        raise RuntimeError(L.sa_last_error().decode())
            reps = max(1, steps // per)
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            return [e0.elapsed_time(e1) / (reps * per)]
        # Ten windows, each exactly `steps` steps between two HIP events on the
        # launch stream.  Each window first runs a GPU-side wait, untimed,
        # long enough for the host to enqueue every step of the window behind
        # it: the steps then run back to back, and the window times the GPU,
        # not the host's launch rate.  (Events between the steps of one window
        # would add their own serialisation: ~1 us per event here.)
        out, done = [], 0
        for _ in range(NUM_WINDOWS):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            hold(2.0 + 0.03 * steps)
            e0.record(stream)
            run(calls_per_step, steps, done)
            e1.record(stream)
            torch.cuda.synchronize()
            done += steps
            out.append(e0.elapsed_time(e1) / steps)
        return out

    paths = {
        "fused": [[c] for c in fused],
        "unfused": [[sparsify, c] for c in listed],
        "dense": [[c] for c in dense],
        "read": [[c] for c in readp],
    }
    # the headline is timed last, after the other paths have brought the
    # clocks to their loaded state
    order = [args.only] if args.only else ["unfused", "dense", "read", "fused"]
    wins = {name: timed(paths[name], args.steps, args.warmup) for name in order}
    ms = {name: float(np.median(w)) for name, w in wins.items()}
    head = args.only or "fused"
    ms_step = ms[head]
    us = ms_step * 1000.0

    verified = verify_headline(sa, torch, rot[0], x, t, y, fused[0]) if head == "fused" else None
    alg_bytes = 2 * D_OUT * nnz + 2 * D_IN + 2 * D_OUT
    if head == "dense":
        alg_bytes = 2 * D_OUT * D_IN + 2 * D_IN + 2 * D_OUT
    elif head == "unfused":
        alg_bytes = 2 * D_OUT * nnz + 2 * D_IN + 2 * D_OUT + 6 * nnz
    achieved = alg_bytes / (us * 1e-6) / 1e9
    traffic = load_traffic(alg_bytes) if head == "fused" else None

    out = {
        "metric": METRIC,
        "value": round(us, 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "accumulate": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama2-7b down_proj W 4096x11008 fp16, batch 1, magnitude threshold "
                        "at 50% sparsity (calibrated), x ~ Laplace(0,1)",
            "d_out": D_OUT, "d_in": D_IN, "batch": 1, "target_sparsity": SPARSITY,
            "threshold": t, "nnz": nnz, "achieved_sparsity": round(1 - nnz / D_IN, 5),
            "path": head, "launch": "hip_graph" if args.graph else "stream",
            "weight_copies": copies, "rotation_bytes": copies * wt0.numel() * 2,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": alg_bytes,
        },
        "windows": {
            "n": len(wins[head]), "steps_each": args.steps,
            "median_us": round(us, 3), "min_us": round(min(wins[head]) * 1000.0, 3),
            "max_us": round(max(wins[head]) * 1000.0, 3),
        },
    }
    if verified is not None:
        out["verified"] = verified
    if "dense" in ms and head != "dense":
        out["dense_gemv_us"] = round(ms["dense"] * 1000.0, 3)
        out["speedup_vs_dense"] = round(ms["dense"] / ms_step, 3)
        dense_bytes = 2 * D_OUT * D_IN + 2 * D_IN + 2 * D_OUT
        out["dense_gemv_frac_of_peak"] = round(
            dense_bytes / (ms["dense"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
    if "unfused" in ms and head != "unfused":
        out["unfused_us"] = round(ms["unfused"] * 1000.0, 3)
    if "read" in ms:
        rgbs = read_bytes / (ms["read"] * 1e-3) / 1e9
        out["read_stream_peak"] = {
            "what": "plain contiguous read of the same byte count (sa_read_stream), same rotation",
            "bytes": read_bytes, "us": round(ms["read"] * 1000.0, 3), "GBps": round(rgbs, 1),
            "frac_of_8TBs": round(rgbs / HBM_PEAK_GBS, 4),
            "headline_frac_of_read_peak": round(achieved / rgbs, 4) if head == "fused" else None,
        }

    out["device"] = device_info(torch, dev)
    if not args.no_cpu_baseline and not args.only:
        out["cpu_baseline"] = cpu_baseline(x_np, t, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    if verified is not None and not verified["ok"]:
        sys.exit(3)


def verify_headline(sa, torch, wt, x, t, y, call):
    """The timed call's output against an fp32 torch product of the same
    thresholded activation (rel. L2 <= 2e-3, max abs <= 1e-2, no NaN), and
    the fused call at t = 0 against the library's dense GEMV."""
    f, a = call
    if f(*a) != 0:
        raise RuntimeError(sa.lib().sa_last_error().decode())
    torch.cuda.synchronize()
    got = y.float().clone()
    keep = (x.float().abs() >= t) & (x != 0)
    ref = torch.where(keep, x.float(), torch.zeros_like(x, dtype=torch.float32)) @ wt.float()
    err = got - ref
    rel = float(torch.linalg.vector_norm(err) / torch.linalg.vector_norm(ref))
    mx = float(err.abs().max())
    dense = sa.dense_gemv(wt, x).float()
    at0 = sa.sparse_gemv_threshold(wt, x, 0.0).float()
    rel0 = float(torch.linalg.vector_norm(at0 - dense) / torch.linalg.vector_norm(dense))
    nan = bool(torch.isnan(got).any())
    ok = (not nan) and rel <= 2e-3 and mx <= 1e-2 and rel0 <= 2e-3
    return {"ok": ok, "against": "fp32 torch product of the thresholded x; t=0 vs dense_gemv",
            "rel_l2": float(f"{rel:.3e}"), "max_abs": float(f"{mx:.3e}"),
            "t0_vs_dense_rel_l2": float(f"{rel0:.3e}"), "nan": nan}


def run_suite(args):
    """Every hot-path row on its workload; one JSON line per measurement.

    HBM-bound kernels rotate their weights over >= 1 GiB of distinct copies;
    times are HIP events around back-to-back calls on the launch stream.
    """
    import torch

    import sparse_input_gemv_amd as sa
    import synthetic as syn

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # Bring the clocks to their loaded steady state before anything is timed:
    # the first fraction of a second of heavy work runs measurably slower.
    wx = torch.from_numpy(syn.gaussian_f16((2048, 4096), 1.0, 1)).to(dev)
    ww = torch.from_numpy(syn.weight_t(4096, 4096, 2)).to(dev)
    wy = torch.empty((2048, 4096), dtype=torch.float16, device=dev)
    t_end = time.time() + 0.5
    while time.time() < t_end:
        for _ in range(50):
            sa.dense_gemm(wx, ww, wy)
        torch.cuda.synchronize()
    del wx, ww, wy

    def ev_time(fn, steps, warmup=20):
        """GPU time per call: `per` calls captured in a HIP graph, replayed.

        The graph removes the Python binding's per-call host cost (output
        allocation, argument checks), which for the smallest kernels would
        otherwise exceed the kernel time.
        """
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        per = min(steps, 24)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(per):
                fn(i)
        reps = max(2, steps // per)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * per) * 1000.0  # us

    def emit(row, name, us, bytes_=None, flops=None, **extra):
        rec = {"row": row, "name": name, "us": round(us, 3)}
        if bytes_ is not None:
            gbs = bytes_ / (us * 1e-6) / 1e9
            rec.update(bytes=int(bytes_), GBps=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4))
        if flops is not None:
            tf = flops / (us * 1e-6) / 1e12
            rec.update(flops=int(flops), TFLOPs=round(tf, 1))
        rec.update(extra)
        print(json.dumps(rec), flush=True)

    def rotation(d_out, d_in, seed):
        w0 = torch.from_numpy(syn.weight_t(d_out, d_in, seed)).to(dev)
        n = max(2, -(-ROTATION_BYTES // (w0.numel() * 2)))
        return [w0] + [torch.roll(w0, shifts=997 * i, dims=0).contiguous() for i in range(1, n)]

    wanted = None if args.rows is None else set(args.rows.split(","))

    def section(*rows):
        return wanted is None or any(r in wanted for r in rows)

    if section("read"):
        suite_read_curve(sa, dev, ev_time, emit)
    if section("config1"):
        suite_single_layer(sa, syn, dev, ev_time, emit)
    # ---- a9 calibration; a1 threshold; a4 / a8 GEMVs of the Llama-2-7B layer ----
    if section("a9", "a1", "a4", "a8", "next1"):
        suite_layer(sa, syn, dev, ev_time, emit, rotation)
    if section("a2", "a5"):
        suite_topk(sa, syn, dev, ev_time, emit, rotation)
    if section("a6", "a8"):
        suite_swiglu(sa, syn, dev, ev_time, emit, rotation)
    if section("a3", "a7", "a8"):
        suite_matmul(sa, syn, dev, ev_time, emit)
    if section("next2"):
        suite_rank_adapter(sa, syn, dev, ev_time, emit)
    if section("next3"):
        suite_corrected(sa, syn, dev, ev_time, emit, rotation)
    if section("next4"):
        suite_shared_nm(sa, syn, dev, ev_time, emit)


def suite_layer(sa, syn, dev, ev_time, emit, rotation):
    import torch

    thresholds = {}
    for inp in syn.LLAMA2_7B_INPUTS:
        smp = torch.from_numpy(syn.calibration_samples(inp)).to(dev)
        us = ev_time(lambda i: sa.act_calibrate_threshold(smp, 0.5), 200)
        thresholds[inp] = {s_: float(sa.act_calibrate_threshold(smp, s_).cpu()[0])
                           for s_ in (0.4, 0.5, 0.6)}
        emit("a9", f"act_calibrate_threshold {inp} n=10000", us, bytes_=2 * 10000)
    layer = {"sparse": 0.0, "dense": 0.0}
    per = {}  # projection -> (sparse us at 50%, dense us)
    for name, (d_out, d_in, inp) in syn.LLAMA2_7B.items():
        _, dist = syn.LLAMA2_7B_INPUTS[inp]
        rot = rotation(d_out, d_in, syn.weight_seed(name))
        nr = len(rot)
        x = torch.from_numpy(syn.activation((d_in,), dist, 0)).to(dev)
        y = torch.empty((d_out,), dtype=torch.float16, device=dev)
        for sp in (0.4, 0.5, 0.6):
            t = thresholds[inp][sp]
            m_, i_, v_, n_ = sa.act_sparsify_threshold(x, t)
            nnz = int(n_.cpu()[0])
            us = ev_time(lambda i: sa.sparse_gemv_threshold(rot[i % nr], x, t, y=y), 1000)
            emit("a4", f"sparse_gemv_threshold {name} {d_out}x{d_in} sparsity {sp}", us,
                 bytes_=2 * d_out * nnz + 2 * d_in + 2 * d_out, flops=2 * d_out * nnz,
                 achieved_sparsity=round(1 - nnz / d_in, 4))
            if sp == 0.5:
                layer["sparse"] += us
                per[name] = [us, 0.0]
                us_l = ev_time(lambda i: sa.sparse_gemv(rot[i % nr], i_, v_, n_, y=y), 1000)
                emit("a4", f"sparse_gemv (list) {name} {d_out}x{d_in} sparsity 0.5", us_l,
                     bytes_=2 * d_out * nnz + 6 * nnz + 2 * d_out)
                us_s = ev_time(lambda i: sa.act_sparsify_threshold(x, t), 1000)
                emit("a1", f"act_sparsify_threshold d={d_in}", us_s,
                     bytes_=2 * d_in + 6 * nnz + d_in // 8 + 4)
        us_d = ev_time(lambda i: sa.dense_gemv(rot[i % nr], x, y=y), 1000)
        layer["dense"] += us_d
        per[name][1] = us_d
        emit("a8", f"dense_gemv {name} {d_out}x{d_in}", us_d,
             bytes_=2 * d_out * d_in + 2 * d_in + 2 * d_out, flops=2 * d_out * d_in)
        del rot
        torch.cuda.empty_cache()
    emit("a4", "Llama-2-7B layer, 7 projections at 50% vs dense (sum of calls)",
         layer["sparse"], speedup_vs_dense=round(layer["dense"] / layer["sparse"], 3),
         dense_us=round(layer["dense"], 3))

    # Llama-3-8B k / v projection: an 8 MB weight, served by the full-K
    # kernel (one workgroup walks all of d_in), batch 1 and 2
    kv = syn.LLAMA3_8B_KV
    d_out, d_in = kv["d_out"], kv["d_in"]
    _, dist = syn.LLAMA2_7B_INPUTS[kv["input"]]
    t = thresholds[kv["input"]][0.5]
    rot = rotation(d_out, d_in, 41)
    nr = len(rot)
    for b in (1, 2):
        xb = torch.from_numpy(syn.activation((b, d_in), dist, 7)).to(dev)
        yb = torch.empty((b, d_out), dtype=torch.float16, device=dev)
        # rows kept by any batch row (the union the kernel reads), from the
        # sparsifier's bitmasks
        words = np.bitwise_or.reduce(np.stack([
            sa.act_sparsify_threshold(xb[r], t)[0].cpu().numpy().view(np.uint32).ravel()
            for r in range(b)]), axis=0)
        rows = int(np.unpackbits(words.view(np.uint8)).sum())
        us = ev_time(lambda i: sa.sparse_gemv_threshold(rot[i % nr], xb, t, y=yb), 1000)
        us_d = ev_time(lambda i: sa.dense_gemv(rot[i % nr], xb, y=yb), 1000)
        emit("a4", f"sparse_gemv_threshold Llama-3-8B k/v {d_out}x{d_in} batch {b} sparsity 0.5", us,
             bytes_=2 * d_out * rows + 2 * b * (d_in + d_out), rows_read=rows,
             speedup_vs_dense=round(us_d / us, 3))
        emit("a8", f"dense_gemv Llama-3-8B k/v {d_out}x{d_in} batch {b}", us_d,
             bytes_=2 * d_out * d_in + 2 * b * (d_in + d_out), flops=2 * b * d_out * d_in)
    del rot
    torch.cuda.empty_cache()

    # shared-input fused projections: one sparsified input, the members'
    # weights side by side (q|k|v, gate|up), one call
    fused = {"sparse": per["o"][0] + per["down"][0], "dense": per["o"][1] + per["down"][1]}
    for name, (members, inp) in syn.LLAMA2_7B_FUSED.items():
        _, dist = syn.LLAMA2_7B_INPUTS[inp]
        w0 = torch.from_numpy(syn.fused_weight_t(name)).to(dev)
        d_in, d_out = w0.shape
        n = max(2, -(-ROTATION_BYTES // (w0.numel() * 2)))
        rot = [w0] + [torch.roll(w0, shifts=997 * i, dims=0).contiguous() for i in range(1, n)]
        nr = len(rot)
        x = torch.from_numpy(syn.activation((d_in,), dist, 0)).to(dev)
        y = torch.empty((d_out,), dtype=torch.float16, device=dev)
        t = thresholds[inp][0.5]
        nnz = int(sa.act_sparsify_threshold(x, t)[3].cpu()[0])
        us = ev_time(lambda i: sa.sparse_gemv_threshold(rot[i % nr], x, t, y=y), 1000)
        sep = sum(per[m][0] for m in members)
        emit("next1", f"fused sparse_gemv_threshold {'|'.join(members)} {d_out}x{d_in} sparsity 0.5",
             us, bytes_=2 * d_out * nnz + 2 * d_in + 2 * d_out, flops=2 * d_out * nnz,
             separate_calls_us=round(sep, 3), speedup_vs_separate=round(sep / us, 3))
        us_d = ev_time(lambda i: sa.dense_gemv(rot[i % nr], x, y=y), 1000)
        emit("next1", f"fused dense_gemv {'|'.join(members)} {d_out}x{d_in}", us_d,
             bytes_=2 * d_out * d_in + 2 * d_in + 2 * d_out, flops=2 * d_out * d_in,
             separate_calls_us=round(sum(per[m][1] for m in members), 3))
        fused["sparse"] += us
        fused["dense"] += us_d
        del rot, w0
        torch.cuda.empty_cache()
    emit("next1", "Llama-2-7B layer with fused q|k|v and gate|up at 50% (4 calls) vs the same "
         "fused dense", fused["sparse"], speedup_vs_fused_dense=round(fused["dense"] / fused["sparse"], 3),
         fused_dense_us=round(fused["dense"], 3),
         speedup_vs_separate_dense=round(layer["dense"] / fused["sparse"], 3))



def suite_read_curve(sa, dev, ev_time, emit):
    """The achievable read rate: a plain read of S bytes (8 MB .. 1 GiB) on
    three grid sizes, each read from a different place of a 2 GiB buffer so
    that no read is served from the 256 MB Infinity Cache, fitted per grid
    to t(S) = t0 + S / BW (least squares)."""
    import torch

    buf = torch.empty(1 << 30, dtype=torch.float16, device=dev).fill_(1.0)  # 2 GiB
    total = buf.numel() * 2
    sizes = [8 << 20, 32 << 20, 128 << 20, 512 << 20, 1 << 30]
    for blocks in (1024, 2048, 4096):
        sink = torch.empty(4 * blocks, dtype=torch.int32, device=dev)
        pts = []
        for size in sizes:
            nrot = max(1, total // size)
            views = [buf[(k * size) // 2:] for k in range(nrot)]
            us = ev_time(lambda i: sa.read_stream(views[i % nrot], size, blocks, sink),
                         max(24, min(400, (4 << 30) // size)), warmup=5)
            pts.append((size, us))
            emit("read", f"read_stream {size >> 20} MiB grid {blocks}x256", us, bytes_=size)
        S = np.array([p[0] for p in pts], dtype=np.float64)
        T = np.array([p[1] for p in pts], dtype=np.float64) * 1e-6
        A = np.stack([np.ones_like(S), S], axis=1)
        (t0, inv_bw), *_ = np.linalg.lstsq(A, T, rcond=None)
        emit("read", f"read_stream fit grid {blocks}x256: t = t0 + bytes / BW", float(t0 * 1e6),
             t0_us=round(float(t0 * 1e6), 3), BW_GBps=round(1.0 / inv_bw / 1e9, 1),
             BW_frac_of_8TBs=round(1.0 / inv_bw / 1e9 / HBM_PEAK_GBS, 4),
             max_rel_residual=round(float(np.max(np.abs(A @ [t0, inv_bw] - T) / T)), 4))
    del buf


def suite_single_layer(sa, syn, dev, ev_time, emit):
    """Single fp16 layer W 1024 x 1024 ~ N(0, 0.02), x ~ N(0, 1), threshold at
    the 50th percentile of |x| (the library's calibration on x itself), seeds
    0..9.  W is 2 MB and stays in cache, so this is a latency point, not an
    HBM-bandwidth one.  rel-L2 is against an fp32 torch product."""
    import torch

    wt = torch.from_numpy(syn.weight_t(1024, 1024, 1000)).to(dev)
    y = torch.empty((1024,), dtype=torch.float16, device=dev)
    for seed in range(10):
        x = torch.from_numpy(syn.gaussian_f16((1024,), 1.0, seed)).to(dev)
        t = float(sa.act_calibrate_threshold(x, 0.5).cpu()[0])
        nnz = int(sa.act_sparsify_threshold(x, t)[3].cpu()[0])
        us = ev_time(lambda i: sa.sparse_gemv_threshold(wt, x, t, y=y), 2000)
        us_d = ev_time(lambda i: sa.dense_gemv(wt, x, y=y), 2000)
        sa.sparse_gemv_threshold(wt, x, t, y=y)
        keep = (x.float().abs() >= t) & (x != 0)
        ref = torch.where(keep, x.float(), torch.zeros_like(x, dtype=torch.float32)) @ wt.float()
        rel = float(torch.linalg.vector_norm(y.float() - ref) / torch.linalg.vector_norm(ref))
        emit("config1", f"sparse_gemv_threshold 1024x1024 seed {seed} (cache-resident latency "
             "point)", us, nnz=nnz, achieved_sparsity=round(1 - nnz / 1024, 4),
             rel_l2=float(f"{rel:.3e}"), dense_gemv_us=round(us_d, 3), threshold=t)


def suite_topk(sa, syn, dev, ev_time, emit, rotation):
    """a2 Top-K and a5 batched union GEMV."""
    import torch

    for d in (4096, 11008):
        d_out = 11008 if d == 4096 else 4096
        rot = rotation(d_out, d, 20 + d)
        nr = len(rot)
        for batch in (1, 2, 4, 8):
            for pct in (60, 50, 40):
                X = torch.from_numpy(syn.laplace_f16((batch, d), 1.0, 100 + batch)).to(dev)
                y = torch.empty((batch, d_out), dtype=torch.float16, device=dev)
                k = syn.topk_k(pct, d)
                m_, i_, v_, n_ = sa.act_sparsify_topk(X, k)
                shifts = torch.arange(32, device=dev, dtype=torch.int32)
                bits = ((m_.unsqueeze(-1) >> shifts) & 1).reshape(batch, -1)[:, :d]
                union = int(torch.count_nonzero(bits.any(0)).cpu())
                us_k = ev_time(lambda i: sa.act_sparsify_topk(X, k), 500)
                emit("a2", f"act_sparsify_topk d={d} K={pct}% batch={batch}", us_k,
                     bytes_=batch * (2 * d + 6 * k + d // 8 + 4))
                us = ev_time(lambda i: sa.sparse_gemv(rot[i % nr], i_, v_, n_, y=y), 500)
                emit("a5" if batch > 1 else "a4", f"sparse_gemv union {d_out}x{d} K={pct}% "
                     f"batch={batch}", us,
                     bytes_=2 * d_out * union + 6 * batch * k + 2 * batch * d_out,
                     flops=2 * d_out * k * batch, union_frac=round(union / d, 4),
                     select_plus_gemv_us=round(us_k + us, 3))
                us_c = ev_time(lambda i: sa.act_topk_cutoff(X, k), 500)
                emit("a2", f"act_topk_cutoff d={d} K={pct}% batch={batch}", us_c,
                     bytes_=batch * (2 * d + 8))
                us_f = ev_time(lambda i: sa.sparse_gemv_topk(rot[i % nr], X, k, y=y), 500)
                try:  # its two-launch form: the select kernel, then the GEMV
                    sa.set_gemv_test_hooks(2)
                    us_2 = ev_time(lambda i: sa.sparse_gemv_topk(rot[i % nr], X, k, y=y), 500)
                finally:
                    sa.set_gemv_test_hooks(0)
                emit("a5" if batch > 1 else "a4", f"sparse_gemv_topk {d_out}x{d} K={pct}% "
                     f"batch={batch} (select + GEMV, no lists)", us_f,
                     bytes_=2 * d_out * union + 2 * batch * d + 8 * batch + 2 * batch * d_out,
                     flops=2 * d_out * k * batch, union_frac=round(union / d, 4),
                     two_launch_us=round(us_2, 3))
        del rot
        torch.cuda.empty_cache()



def suite_corrected(sa, syn, dev, ev_time, emit, rotation):
    """Weight-aware selection with the static shift and the variance
    correction on the down projection (4096 x 11008): the scored sparsifier
    then the corrected list GEMV, against the plain fused threshold call."""
    import torch

    d_out, d_in, inp = syn.LLAMA2_7B["down"]
    _, dist = syn.LLAMA2_7B_INPUTS[inp]
    rot = rotation(d_out, d_in, syn.weight_seed("down"))
    nr = len(rot)
    x = torch.from_numpy(syn.activation((d_in,), dist, 0)).to(dev)
    mu = torch.from_numpy(syn.gaussian_f16((d_in,), 0.25, 13)).to(dev)
    cn = sa.weight_col_norms(rot[0])
    bias = sa.dense_gemv(rot[0], mu)
    y = torch.empty((d_out,), dtype=torch.float16, device=dev)
    xs = (x.float() - mu.float()).half().double().abs()
    sc = torch.sort(xs * cn).values
    t = float(0.5 * (sc[d_in // 2 - 1] + sc[d_in // 2]))
    t_plain = float(torch.sort(x.float().abs()).values[d_in // 2])
    us_p = ev_time(lambda i: sa.sparse_gemv_threshold(rot[i % nr], x, t_plain, y=y), 1000)
    kept_f = int((sc >= t).sum())
    us_f = ev_time(lambda i: sa.sparse_gemv_scored(rot[i % nr], x, t, mu=mu, colnorm=cn, var=True,
                                                   bias=bias, y=y), 1000)
    emit("next3", f"sparse_gemv_scored down {d_out}x{d_in} weight-aware threshold 50%, shift + "
         "VAR, one launch", us_f,
         bytes_=2 * d_out * kept_f + 2 * d_in * 2 + 8 * d_in + 2 * d_out * 2,
         flops=2 * d_out * kept_f, kept=kept_f, plain_fused_us=round(us_p, 3))
    for label, (tt, n, m) in (("threshold 50%", (t, 0, 0)), ("8:16", (0.0, 8, 16))):
        out = sa.act_sparsify_scored(x, t=tt, n=n, m=m, mu=mu, colnorm=cn, with_mask=False)
        _, idx, val, nnz, alpha = out
        kept = int(nnz.cpu()[0])
        us_s = ev_time(lambda i: sa.act_sparsify_scored(x, t=tt, n=n, m=m, mu=mu, colnorm=cn,
                                                        with_mask=False), 1000)
        us_g = ev_time(lambda i: sa.sparse_gemv_corrected(rot[i % nr], idx, val, nnz, alpha=alpha,
                                                          bias=bias, y=y), 1000)
        emit("next3", f"act_sparsify_scored + sparse_gemv_corrected down {d_out}x{d_in} "
             f"weight-aware {label}, shift + VAR", us_s + us_g,
             bytes_=2 * d_out * kept + 6 * kept + 2 * d_in * 2 + 8 * d_in + 2 * d_out * 2,
             flops=2 * d_out * kept, kept=kept, sparsify_us=round(us_s, 3), gemv_us=round(us_g, 3),
             plain_fused_us=round(us_p, 3))
    for (n, m) in ((8, 16), (16, 32)):
        kept = d_in // m * n
        us_n = ev_time(lambda i: sa.sparse_gemv_scored_nm(rot[i % nr], x, n, m, mu=mu, colnorm=cn,
                                                          var=True, bias=bias, y=y), 1000)
        emit("next3", f"sparse_gemv_scored_nm down {d_out}x{d_in} weight-aware {n}:{m}, shift + "
             "VAR, one launch", us_n,
             bytes_=2 * d_out * kept + 2 * d_in * 2 + 8 * d_in + 2 * d_out * 2,
             flops=2 * d_out * kept, kept=kept, plain_fused_us=round(us_p, 3))
    del rot
    torch.cuda.empty_cache()


def suite_rank_adapter(sa, syn, dev, ev_time, emit):
    """RaNA linear-layer rank adapter A (m ⊙ B x) on the gate projection
    (11008 x 4096) at rank 2048, 50% mask rate, against the dense gate GEMV."""
    import torch

    d_out, d_in, r = 11008, 4096, 2048
    bt0, at0 = (torch.from_numpy(w).to(dev) for w in syn.rank_adapter_weights(d_out, d_in, r, 3000))
    b0 = bt0.t().contiguous()  # B [r][d_in], row-major
    pair = (b0.numel() + at0.numel()) * 2
    n = max(2, -(-ROTATION_BYTES // pair))
    # copy i permutes the rank index (B's rows and A's rows of A^T alike):
    # other bytes in memory, the same adapter, mask size and y
    rot = [(b0, at0)] + [(torch.roll(b0, 97 * i, 0).contiguous(),
                          torch.roll(at0, 97 * i, 0).contiguous()) for i in range(1, n)]
    wt_gate = torch.from_numpy(syn.weight_t(d_out, d_in, syn.weight_seed("gate"))).to(dev)
    ng = max(2, -(-ROTATION_BYTES // (wt_gate.numel() * 2)))
    rot_g = [wt_gate] + [torch.roll(wt_gate, 997 * i, 0).contiguous() for i in range(1, ng)]
    x = torch.from_numpy(syn.activation((d_in,), "gaussian", 0)).to(dev)
    v = torch.empty((r,), dtype=torch.float16, device=dev)
    y = torch.empty((d_out,), dtype=torch.float16, device=dev)
    nr = len(rot)
    sq = torch.sort(sa.rana_adapter_gemv(b0, at0, x, 0.0)[0].double() ** 2).values
    for rate in (0.5, 0.7):
        k = int(rate * r)
        t = float(0.5 * (sq[k - 1] + sq[k]))
        kept = int((sq >= t).sum())
        us = ev_time(lambda i: sa.rana_adapter_gemv(rot[i % nr][0], rot[i % nr][1], x, t, v=v, y=y),
                     1000)
        bytes_ = 2 * d_in * r + 2 * d_out * kept + 2 * d_in + 2 * 2 * r + 2 * d_out
        us_d = ev_time(lambda i: sa.dense_gemv(rot_g[i % len(rot_g)], x, y=y), 1000)
        emit("next2", f"rana_adapter_gemv gate {d_out}x{d_in} rank {r} mask rate {rate}", us,
             bytes_=bytes_, flops=2 * d_in * r + 2 * d_out * kept, kept=kept,
             dense_gate_us=round(us_d, 3), speedup_vs_dense_gate=round(us_d / us, 3))
    del rot, rot_g
    torch.cuda.empty_cache()


def suite_swiglu(sa, syn, dev, ev_time, emit, rotation):
    """a6 masked SwiGLU down projection (Llama-3-8B MLP)."""
    import torch

    d_model, d_ff = syn.LLAMA3_8B_MLP["d_model"], syn.LLAMA3_8B_MLP["d_ff"]
    rot = rotation(d_model, d_ff, 31)
    nr = len(rot)
    g, u = (torch.from_numpy(a).to(dev) for a in syn.swiglu_gate_up(d_ff, d_model, 0))
    cn = [sa.weight_col_norms(w) for w in rot[:1]][0]
    y = torch.empty((d_model,), dtype=torch.float16, device=dev)
    x_dense = torch.from_numpy(syn.gaussian_f16((d_ff,), 1.0, 0)).to(dev)
    us_d = ev_time(lambda i: sa.dense_gemv(rot[i % nr], x_dense, y=y), 500)
    emit("a8", f"dense_gemv down {d_model}x{d_ff}", us_d, bytes_=2 * d_model * d_ff + 2 * d_ff + 2 * d_model)
    # the MLP's two dense projections (gate, up: d_ff x d_model), for the MLP totals
    rot_gu = rotation(d_ff, d_model, 32)
    x_in = torch.from_numpy(syn.gaussian_f16((d_model,), 1.0, 1)).to(dev)
    y_ff = torch.empty((d_ff,), dtype=torch.float16, device=dev)
    us_gu = ev_time(lambda i: sa.dense_gemv(rot_gu[i % len(rot_gu)], x_in, y=y_ff), 500)
    emit("a8", f"dense_gemv gate/up {d_ff}x{d_model}", us_gu,
         bytes_=2 * d_model * d_ff + 2 * d_ff + 2 * d_model)
    del rot_gu
    mlp_dense = 2 * us_gu + us_d
    for mode in ("cats", "rana"):
        for rate in (0.5, 0.7):
            # threshold at the score quantile of this draw (the library's own calibration)
            if mode == "cats":
                sc = torch.abs(torch.nn.functional.silu(g.double()))
            else:
                sc = torch.abs(torch.nn.functional.silu(g.double()) * u.double()) * cn
            t = float(torch.quantile(sc.cpu(), rate))
            yy, mk, nz = sa.masked_swiglu_down(g, u, rot[0], t, mode, cn if mode == "rana" else None)
            nnz = int(nz.cpu()[0])
            us = ev_time(lambda i: sa.masked_swiglu_down(g, u, rot[i % nr], t, mode,
                                                          cn if mode == "rana" else None, y=y,
                                                          with_mask=False), 500)
            extra = 8 * d_ff if mode == "rana" else 0
            emit("a6", f"masked_swiglu_down {mode} mask rate {rate}", us,
                 bytes_=2 * d_model * nnz + 4 * d_ff + extra + 2 * d_model, flops=2 * d_model * nnz,
                 kept=nnz, speedup_vs_dense_down=round(us_d / us, 3))
            emit("a6", f"Llama-3-8B MLP: dense gate + up, {mode} masked down at {rate} "
                 "vs the dense MLP (sum of calls)", 2 * us_gu + us, dense_mlp_us=round(mlp_dense, 3),
                 speedup_vs_dense_mlp=round(mlp_dense / (2 * us_gu + us), 3))
    us_c = ev_time(lambda i: sa.weight_col_norms(rot[i % nr]), 50)
    emit("a6", f"weight_col_norms {d_ff}x{d_model}", us_c, bytes_=2 * d_ff * d_model + 8 * d_ff)
    del rot
    torch.cuda.empty_cache()



def suite_matmul(sa, syn, dev, ev_time, emit):
    """a3 N:M sparsify, a7 N:M matmul, a8 dense GEMM.  MFMA fractions price
    algorithmic FLOPs against the dense fp16 peak, also for 2:4."""
    import torch

    # the two configured shapes (every pattern, with the sparsifier), then
    # two where the dense engine takes 256 x 256 tiles (one and 2.7 tiles
    # per CU)
    for (T, d_in, d_out, full) in [(4096, 1024, 1024, True), (2048, 4096, 11008, True),
                                   (4096, 4096, 4096, False), (4096, 4096, 11008, False)]:
        X = torch.from_numpy(syn.gaussian_f16((T, d_in), 1.0, 5)).to(dev)
        wt = torch.from_numpy(syn.weight_t(d_out, d_in, 41)).to(dev)
        y = torch.empty((T, d_out), dtype=torch.float16, device=dev)
        dense_flop = 2 * T * d_in * d_out
        steps = 200 if T * d_in * d_out < 1e10 else 30
        us_g = ev_time(lambda i: sa.dense_gemm(X, wt, y=y), steps, warmup=3)
        emit("a8", f"dense_gemm {T}x{d_in}x{d_out}", us_g, flops=dense_flop,
             frac_mfma=round(dense_flop / (us_g * 1e-6) / 2.5e15, 4))
        for (n, m) in ([(2, 4), (8, 16), (16, 32)] if full else [(2, 4), (8, 16)]):
            mask, val = sa.act_sparsify_nm(X, n, m)
            if full:
                us_s = ev_time(lambda i: sa.act_sparsify_nm(X, n, m), 200)
                emit("a3", f"act_sparsify_nm {n}:{m} {T}x{d_in}", us_s,
                     bytes_=2 * T * d_in + 2 * T * d_in * n // m + T * d_in // 8)
            us = ev_time(lambda i: sa.nm_act_spmm(val, mask, n, m, wt, y=y), steps, warmup=3)
            alg = dense_flop * n // m
            emit("a7", f"nm_act_spmm {n}:{m} {T}x{d_in}x{d_out}", us, flops=alg,
                 frac_mfma=round(alg / (us * 1e-6) / 2.5e15, 4),
                 speedup_vs_dense_gemm=round(us_g / us, 3))


def suite_shared_nm(sa, syn, dev, ev_time, emit):
    """Tile-shared N:M: one pattern per tile of tt tokens (VW32 is tt = 32),
    sparsify and matmul, against the dense GEMM of the same shape.  Algorithmic
    FLOPs are the kept columns' (n/m of dense), priced against the dense fp16
    peak."""
    import torch

    for (T, d_in, d_out) in [(4096, 1024, 1024), (2048, 4096, 11008)]:
        X = torch.from_numpy(syn.gaussian_f16((T, d_in), 1.0, 5)).to(dev)
        wt = torch.from_numpy(syn.weight_t(d_out, d_in, 41)).to(dev)
        y = torch.empty((T, d_out), dtype=torch.float16, device=dev)
        dense_flop = 2 * T * d_in * d_out
        steps = 200 if T * d_in * d_out < 1e10 else 30
        us_g = ev_time(lambda i: sa.dense_gemm(X, wt, y=y), steps, warmup=3)
        for tt in (32, 128, 256):
            for (n, m) in [(8, 16), (16, 32), (2, 4), (1, 4), (4, 16)]:
                if tt == 256 and (n, m) not in ((8, 16), (1, 4)):
                    continue
                mask, val = sa.act_sparsify_nm_shared(X, n, m, tt)
                if (n, m) == (8, 16):
                    us_s = ev_time(lambda i: sa.act_sparsify_nm_shared(X, n, m, tt), 200)
                    emit("next4", f"act_sparsify_nm_shared {n}:{m} tt={tt} {T}x{d_in}", us_s,
                         bytes_=2 * T * d_in + 2 * T * d_in * n // m + -(-T // tt) * d_in // 8)
                us = ev_time(lambda i: sa.nm_shared_spmm(val, mask, n, m, tt, wt, y=y), steps,
                             warmup=3)
                alg = dense_flop * n // m
                emit("next4", f"nm_shared_spmm {n}:{m} tt={tt} {T}x{d_in}x{d_out}", us, flops=alg,
                     frac_mfma=round(alg / (us * 1e-6) / 2.5e15, 4),
                     speedup_vs_dense_gemm=round(us_g / us, 3), dense_gemm_us=round(us_g, 3))


def _oracle_step(wt, x, t):
    from oracle import gemv, sparsify

    keep, idx, val, nnz = sparsify.threshold_sparsify(x, t)
    return gemv.sparse_gemv(wt, idx, val)


def _cpu_worker(args):
    """One process of the all-cores run: its own copy of the inputs (drawn
    from the same seeds), then oracle steps until the shared end time."""
    t, start, end = args
    from threadpoolctl import threadpool_limits

    import synthetic as syn

    wt = syn.weight_t(D_OUT, D_IN, syn.weight_seed("down"))
    x = syn.activation((D_IN,), "laplace", 0)
    calls = 0
    with threadpool_limits(limits=1):
        while time.time() < start:
            time.sleep(0.01)
        while time.time() < end:
            _oracle_step(wt, x, t)
            calls += 1
    return calls


def device_info(torch, dev):
    """The GPU, its runtime and the host the line was measured on."""
    pr = torch.cuda.get_device_properties(dev)
    return {
        "name": pr.name, "arch": getattr(pr, "gcnArchName", None),
        "compute_units": pr.multi_processor_count,
        "hbm_gib": round(pr.total_memory / 2**30, 1),
        "hip_runtime": getattr(torch.version, "hip", None), "torch": torch.__version__,
        "host_cpu": _cpu_model(), "host_nproc": _nproc(),
    }


def _nproc():
    """Cores this process may run on (its affinity set), as nproc counts them."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(x, t, seconds):
    """The oracle (fp64 numpy, as it stands) on the headline step: one
    thread, then one process per host core (at most 16, the share of one
    GPU) running steps side by side; the all-cores figure is wall time per
    step of the aggregate throughput."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits

    import synthetic as syn

    wt = syn.weight_t(D_OUT, D_IN, syn.weight_seed("down"))
    calls, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=1):
        while True:
            _oracle_step(wt, x, t)
            calls += 1
            el = time.perf_counter() - t0
            if el >= seconds / 2 or calls >= 100:
                break
    single_us = el / calls * 1e6
    del wt
    ncpu = _nproc()
    procs = max(1, min(ncpu, 16))
    window = seconds / 2
    ctx = mp.get_context("spawn")
    with ctx.Pool(procs) as pool:
        start = time.time() + 8.0  # every worker has its inputs by then
        end = start + window
        total = sum(pool.map(_cpu_worker, [(t, start, end)] * procs))
    all_us = window / max(total, 1) * 1e6
    return {
        "value": round(all_us, 1), "unit": "us", "cores": procs, "kind": "oracle",
        "sample": f"the full headline step (threshold + sparse GEMV, 4096x11008, 50%) in fp64 "
                  f"numpy: {procs} processes side by side for {window:.1f} s ({total} steps; "
                  f"value = window / steps), and {calls} steps on one thread in {el:.1f} s",
        "single_thread_us": round(single_us, 1), "nproc": ncpu, "cpu_model": _cpu_model(),
    }


if __name__ == "__main__":
    main()
