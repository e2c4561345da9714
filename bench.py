"""Benchmark of the ring-attention rank view on one MI355X.

One step = the whole hot path over one batch of the workload: the layout gather of K/V into
ring order, and for every rank view of the workload the gather of its Q and dO slices, the
forward ring loop (staged K/V, chunk kernels, finalize) and, where the workload has it, the
backward ring loop (delta pre-pass, staged K/V, chunk kernels, casts).

Prints one JSON line.  `value` is attention TFLOP/s over the timed steps, counting only
unmasked work: 4*D*Lq*Lkv per full pair and 2*D*L^2 per diagonal pair, times B*Hq, for the
forward; 2.5x that for the backward (five contractions including the recompute).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "attention TFLOP/s fwd+bwd per rank view at 1 GPU; % of bf16 MFMA peak"
DEFAULT_WORKLOAD = "long-ring-cp16-zigzag"
# also timed (rank views only, fewer steps) and reported beside the headline
EXTRA_WORKLOADS = ("long-ring-cp16-contiguous", "llama-gqa-cp8-zigzag")


def visible_count(q_pos0, kv_pos0, q_len, kv_len, window, attn_chunk):
    """Number of visible (query, key) pairs of a pair block under the causal mask restricted by
    a sliding window and / or attention chunks (positions are consecutive in both ranges)."""
    import numpy as np
    t = np.arange(q_pos0, q_pos0 + q_len, dtype=np.int64)
    hi = np.minimum(t, kv_pos0 + kv_len - 1)
    lo = np.full_like(t, kv_pos0)
    if window:
        lo = np.maximum(lo, t - window + 1)
    if attn_chunk:
        lo = np.maximum(lo, (t // attn_chunk) * attn_chunk)
    return int(np.maximum(hi - lo + 1, 0).sum())


def counted_flops(api, prob, rank):
    """Forward FLOPs of one rank view by the metric's counting rule (per ring step): 4 d L^2 per
    full pair and 2 d L^2 per diagonal pair; with a sliding window or attention chunks, 4 d per
    visible (query, key) pair."""
    per_step = []
    masked = bool(prob.window or prob.attn_chunk)
    for i in range(prob.cp):
        _, pairs = api.ra_plan_step(prob, rank, i, positions=True)
        f = 0
        for q0, k0, ql, kl, mask, qp0, kp0 in pairs:
            if mask == 2:
                continue
            if masked:
                f += 4 * prob.head_dim * visible_count(qp0, kp0, ql, kl, prob.window, prob.attn_chunk)
            elif mask == 0:
                f += 4 * prob.head_dim * ql * kl
            else:
                f += 2 * prob.head_dim * ql * kl
        per_step.append(f * prob.batch * prob.heads_q)
    return per_step


def cpu_baseline(wl, t, target_s: float):
    """The FP64 oracle on a bounded sample of rank 0's rows, as a TFLOP/s rate."""
    import numpy as np
    from oracle import attn64 as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                      or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    rank = wl.ranks[0]
    pos = O.rank_positions(wl.seq_len, wl.cp, wl.layout, rank)
    n_rep = wl.heads_q // wl.heads_kv
    kpos = np.arange(wl.seq_len)
    q_all, k_all, v_all, do_all = (t.as_f64(n)[:1] for n in ("q", "k", "v", "do"))

    # rows from the end of the slice (the rows with the most visible keys), then more key/value
    # groups (each with its n_rep query heads) until the sample takes about target_s
    def run(nrows, ngroups):
        rows = pos[-nrows:]
        t0 = time.perf_counter()
        for g in range(ngroups):
            heads = list(range(g * n_rep, (g + 1) * n_rep))
            q, do = q_all[:, heads][:, :, rows], do_all[:, heads][:, :, rows]
            k, v = k_all[:, g:g + 1], v_all[:, g:g + 1]
            O.attention_rows(q, k, v, rows, kpos)
            O.attention_rows_bwd(q, k, v, do, rows, kpos)
        dt = time.perf_counter() - t0
        vis = float(np.sum(rows + 1))  # keys visible to each row (causal, full sequence)
        flops = (4 + 10) * wl.head_dim * vis * n_rep * ngroups
        return dt, flops, rows

    n, g = 16, 1
    dt, flops, rows = run(n, g)
    while dt < target_s / 8 and n < len(pos):
        n = min(len(pos), n * 4)
        dt, flops, rows = run(n, g)
    if dt < target_s / 2 and n < len(pos):
        n = min(len(pos), int(n * target_s / max(dt, 1e-3) * 0.8))
        dt, flops, rows = run(n, g)
    if dt < target_s / 2 and n == len(pos) and wl.heads_kv > 1:
        g = min(wl.heads_kv, max(2, int(target_s / max(dt, 1e-3) * 0.8)))
        dt, flops, rows = run(n, g)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"rank {rank} of {wl.name}: last {len(rows)} rows of the Q slice x {g * n_rep} "
                      f"query heads ({g} key/value group(s)), forward + backward over the full causal "
                      f"key prefix, FP64, {dt:.1f} s"}


def chunk_launches(api, prob, wl, k_ring, v_ring):
    """The chunk-kernel launches of every rank view of the workload: (rank, pairs, k, v, fwd FLOPs)."""
    chunk = prob.chunk
    out = []
    for r in wl.ranks:
        flops = counted_flops(api, prob, r)
        for i in range(prob.cp):
            owner, pairs = api.ra_plan_step(prob, r, i, positions=True)
            if all(p[4] == 2 for p in pairs):
                continue
            kc = k_ring[:, :, owner * chunk:(owner + 1) * chunk].contiguous()
            vc = v_ring[:, :, owner * chunk:(owner + 1) * chunk].contiguous()
            out.append((r, pairs, kc, vc, flops[i]))
    return out


# Algorithmic FLOPs of each chunk kernel per unit of counted forward FLOPs (the metric's method
# work): the forward does Q K^T and P V (1); the dK/dV kernel S, dP, dV and dK (2); the dQ kernel
# of the rank views forms dQ from the stored dS (0.5).  Together: the backward's 2.5.
KERNEL_UNITS = {"chunk_fwd_pp_kernel": 1.0, "chunk_bwd_kv_pp_kernel": 2.0, "chunk_bwd_dq_ds_kernel": 0.5}


def kernel_runners(api, ctx, prob, wl, bufs, launches, stream, backward):
    """One callable per chunk kernel, each launching exactly that kernel for a launch tuple: the
    backward through ra_chunk_bwd_ds in its two phases (dK/dV storing dS, then dQ from it)."""
    import torch
    chunk = prob.chunk
    U, m, l = api.new_state(prob, chunk)
    api.ra_state_init(ctx, prob, U, m, l)
    run = {"chunk_fwd_pp_kernel": lambda L: api.ra_chunk_fwd(
        ctx, prob, bufs[L[0]]["q"], L[2], L[3], L[1], U, m, l, stream)}
    if backward:
        delta = {r: api.ra_bwd_preprocess(ctx, prob, bufs[r]["o"], bufs[r]["do"]) for r in wl.ranks}
        dq = torch.zeros((prob.batch, prob.heads_q, chunk, prob.head_dim), device="cuda")
        dk = torch.zeros((prob.batch, prob.heads_kv, chunk, prob.head_dim), device="cuda")
        dv = torch.zeros_like(dk)
        nbytes = max(api.ra_chunk_bwd_ds_size(prob, chunk, chunk, L[1]) for L in launches)
        scratch = torch.empty(max(16, nbytes), dtype=torch.uint8, device="cuda")
        b = lambda L: bufs[L[0]]
        run["chunk_bwd_kv_pp_kernel"] = lambda L: api.ra_chunk_bwd_ds(
            ctx, prob, b(L)["q"], b(L)["do"], b(L)["lse"], delta[L[0]], L[2], L[3], L[1], None, dk, dv,
            scratch, stream)
        run["chunk_bwd_dq_ds_kernel"] = lambda L: api.ra_chunk_bwd_ds(
            ctx, prob, b(L)["q"], b(L)["do"], b(L)["lse"], delta[L[0]], L[2], L[3], L[1], dq, None, None,
            scratch, stream)
    return run


def kernel_rates(api, ctx, prob, wl, bufs, launches, stream, backward, reps=3):
    """Average launch duration of each chunk kernel over the workload's launches, timed with
    HIP events on the launch stream, and its algorithmic rate (method work, KERNEL_UNITS).
    The dQ kernel reads the dS its launch's dK/dV phase stored, so the two backward phases are
    replayed launch by launch, each phase bracketed by its own events."""
    import torch
    run = kernel_runners(api, ctx, prob, wl, bufs, launches, stream, backward)
    names = list(run)
    times = {n: [0.0] * len(launches) for n in names}
    ev = {n: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in launches] for n in names}
    for rep in range(reps + 1):  # the first pass warms up
        for j, L in enumerate(launches):
            for n in names:
                ev[n][j][0].record(stream)
                run[n](L)
                ev[n][j][1].record(stream)
        torch.cuda.synchronize()
        if rep == 0:
            continue
        for n in names:
            for j in range(len(launches)):
                times[n][j] += ev[n][j][0].elapsed_time(ev[n][j][1]) / reps
    out = {}
    for name in names:
        flops = KERNEL_UNITS[name] * sum(L[4] for L in launches) / len(launches)
        avg_ms = sum(times[name]) / len(launches)
        out[name] = {"avg_launch_ms": round(avg_ms, 4), "launches": len(launches),
                     "algorithmic_tflop_per_launch": round(flops / 1e12, 5),
                     "achieved_tflops": round(flops / (avg_ms * 1e-3) / 1e12, 2),
                     "frac": round(flops / (avg_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                     "total_ms_per_pass": round(sum(times[name]), 4)}
    return out


# The files the chunk kernels' code and parameter block come from: the stored counter readings
# describe these kernels and stay valid while these files do.
CHUNK_KERNEL_SOURCES = ("kern_bwd.hip", "kern_common.h", "kern_fwd.hip", "ra_internal.h", "ra_host.cpp",
                        "ra_plan.cpp")


def source_hash():
    """Hash of the chunk kernels' sources: stored counter readings are used only while it matches."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "context_blockwise_causal_amd", "csrc")
    for f in CHUNK_KERNEL_SOURCES:
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def traffic_path(wl_name):
    return os.path.join(ROOT, "profiles", f"hbm_traffic_chunk_kernels_{wl_name}.json")


def stored_traffic(wl_name, kernel):
    """HBM bytes per launch of `kernel` from the stored counter readings, if they were taken
    on the current kernel sources; else None."""
    try:
        rec = json.load(open(traffic_path(wl_name)))
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != source_hash() or kernel not in rec.get("kernels", {}):
        return None
    k = rec["kernels"][kernel]
    return k["fetch_bytes_per_launch"] + k["write_bytes_per_launch"]


def traffic_summary(wl_name, fetch_dir, write_dir, calib_bytes, stage_bytes):
    """Turns two rocprofv3 --pmc runs of `--kernels-only` (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch) into bytes per launch, scaled by what the counters read for a calibration copy of
    known size: the last layout-kernel dispatch of the run, which gathers one K tensor (calib_bytes
    read and written).  (The run's earlier layout dispatches gather tensors of other sizes.)  The
    staging copies (copy2d_kernel, stage_bytes read and written per dispatch, a different kernel and
    size) give a second, independent factor; the record keeps both."""
    import csv
    import glob
    import re

    def per_dispatch(root, counter):
        acc = {}
        for f in glob.glob(os.path.join(root, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                m = re.search(r"(chunk_\w+|layout_kernel|copy2d_kernel)", r["Kernel_Name"])
                if not m:
                    continue
                a = acc.setdefault(m.group(1), {})
                d = int(r["Dispatch_Id"])
                a[d] = a.get(d, 0.0) + float(r["Counter_Value"]) * 1024
        return acc

    def avg(d):
        return sum(d.values()) / len(d)

    fetch, write = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    cal_f = fetch["layout_kernel"][max(fetch["layout_kernel"])]
    cal_w = write["layout_kernel"][max(write["layout_kernel"])]
    fs, ws = calib_bytes / cal_f, calib_bytes / cal_w
    rec = {"workload": wl_name, "source_hash": source_hash(),
           "calibration": {"kernel": "layout_kernel (last dispatch: the gather of one K tensor)",
                           "bytes_each_way": calib_bytes, "fetch_read": cal_f, "write_read": cal_w,
                           "fetch_scale": fs, "write_scale": ws},
           "kernels": {k: {"fetch_bytes_per_launch": avg(fetch[k]) * fs, "write_bytes_per_launch": avg(write[k]) * ws,
                           "launches": len(fetch[k])}
                       for k in fetch if k.startswith("chunk_") and k in write}}
    if "copy2d_kernel" in fetch and "copy2d_kernel" in write:
        rec["check"] = {"kernel": "copy2d_kernel", "bytes_each_way": stage_bytes,
                        "fetch_read": avg(fetch["copy2d_kernel"]), "write_read": avg(write["copy2d_kernel"]),
                        "fetch_scale": stage_bytes / avg(fetch["copy2d_kernel"]),
                        "write_scale": stage_bytes / avg(write["copy2d_kernel"])}
    with open(traffic_path(wl_name), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' rank views")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--same-stream", action="store_true", help="stage K/V on the compute stream")
    ap.add_argument("--window", type=int, default=0, help="sliding window (0 = plain causal)")
    ap.add_argument("--attn-chunk", type=int, default=0, help="attention chunk (0 = off)")
    ap.add_argument("--kernels-only", action="store_true",
                    help="only replay the chunk-kernel launches (and one layout gather of K as the "
                         "calibration copy): the program to run under rocprofv3 --pmc")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the stored HBM-traffic record from two rocprofv3 --pmc output "
                         "folders of --kernels-only (FETCH_SIZE, WRITE_SIZE)")
    args = ap.parse_args()
    if args.traffic_summary:
        from context_blockwise_causal_amd.workloads import WORKLOADS
        wl = WORKLOADS[args.workload]
        esize = 2 if wl.dtype == "bf16" else 4
        traffic_summary(wl.name, args.traffic_summary[0], args.traffic_summary[1],
                        wl.batch * wl.heads_kv * wl.seq_len * wl.head_dim * esize,
                        wl.batch * wl.heads_kv * (wl.seq_len // wl.cp) * wl.head_dim * esize)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs a single rank view at a time on one "
              "MI355X (the ring is simulated on one device); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from context_blockwise_causal_amd import api
    from context_blockwise_causal_amd.inputs import draw
    from context_blockwise_causal_amd.workloads import WORKLOADS

    ctx = api.Context(0)
    compute = torch.cuda.current_stream()
    draws = {}

    def drawn(wl):
        key = (wl.batch, wl.seq_len, wl.heads_q, wl.heads_kv, wl.head_dim, wl.dtype, wl.seed)
        if key not in draws:
            draws.clear()
            draws[key] = draw(*key, with_grad=True)
        return draws[key]

    def timed_each(fn, reps, warm=1):
        """Median and all durations (ms) of `reps` calls of fn, each bracketed by events on the
        compute stream."""
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record(compute)
            fn()
            b.record(compute)
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) for a, b in ev]
        return statistics.median(ts), ts

    def workload(name, window=0, attn_chunk=0):
        """Device buffers and the step functions of one workload (allocated outside timing)."""
        wl = WORKLOADS[name]
        prob = api.Problem(wl.batch, wl.seq_len, wl.heads_q, wl.heads_kv, wl.head_dim, wl.cp,
                           wl.layout, wl.dtype, 0.0, window, attn_chunk)
        t = drawn(wl)
        dev = {n: api.to_device(t.store[n], wl.dtype) for n in ("q", "k", "v", "do")}
        staging = compute if args.same_stream else torch.cuda.Stream()
        k_ring = torch.empty_like(dev["k"])
        v_ring = torch.empty_like(dev["v"])
        bufs = {}
        for r in wl.ranks:
            q_sl = torch.empty((wl.batch, wl.heads_q, prob.chunk, wl.head_dim), dtype=prob.torch_dtype,
                               device="cuda")
            bufs[r] = dict(q=q_sl, do=torch.empty_like(q_sl), o=torch.empty_like(q_sl),
                           lse=torch.empty(q_sl.shape[:3], dtype=torch.float32, device="cuda"),
                           dq=torch.empty_like(q_sl), dk=torch.empty_like(k_ring), dv=torch.empty_like(v_ring))
        ws_fwd = api.workspace(prob, 0)
        ws_bwd = api.workspace(prob, 1) if wl.backward else None

        def fwd(r):
            b = bufs[r]
            api.ra_rank_view_fwd(ctx, prob, r, b["q"], k_ring, v_ring, b["o"], b["lse"], ws_fwd,
                                 compute, staging)

        def bwd(r):
            b = bufs[r]
            api.ra_rank_view_bwd(ctx, prob, r, b["q"], k_ring, v_ring, b["o"], b["lse"], b["do"],
                                 b["dq"], b["dk"], b["dv"], ws_bwd, compute, staging)

        def gathers():
            api.ra_layout_gather(ctx, prob, 0, wl.cp, dev["k"], k_ring)
            api.ra_layout_gather(ctx, prob, 0, wl.cp, dev["v"], v_ring)
            for r in wl.ranks:
                api.ra_layout_gather(ctx, prob, r, 1, dev["q"], bufs[r]["q"])
                if wl.backward:
                    api.ra_layout_gather(ctx, prob, r, 1, dev["do"], bufs[r]["do"])

        def step():
            gathers()
            for r in wl.ranks:
                fwd(r)
                if wl.backward:
                    bwd(r)

        fwd_flops = sum(sum(counted_flops(api, prob, r)) for r in wl.ranks)
        return dict(wl=wl, prob=prob, t=t, dev=dev, k_ring=k_ring, v_ring=v_ring, bufs=bufs, fwd=fwd,
                    bwd=bwd, step=step, gathers=gathers, fwd_flops=fwd_flops)

    def rates(W, steps, warmup):
        """Step (fwd+bwd over every rank view) and per-pass medians, counted TFLOP/s."""
        wl = W["wl"]
        ff = W["fwd_flops"]
        total = ff * (3.5 if wl.backward else 1.0)
        for _ in range(warmup):
            W["step"]()
        step_ms, step_all = timed_each(W["step"], steps, warm=0)
        fwd_ms, _ = timed_each(lambda: [W["fwd"](r) for r in wl.ranks], max(3, steps))
        out = {"ms_per_step": step_ms, "step_ms_all": [round(x, 4) for x in step_all],
               "tflops": total / (step_ms * 1e-3) / 1e12, "counted_tflop_per_step": total / 1e12,
               "fwd_ms": fwd_ms, "fwd_tflops": ff / (fwd_ms * 1e-3) / 1e12}
        if wl.backward:
            bwd_ms, _ = timed_each(lambda: [W["bwd"](r) for r in wl.ranks], max(3, steps))
            out["bwd_ms"] = bwd_ms
            out["bwd_tflops"] = 2.5 * ff / (bwd_ms * 1e-3) / 1e12
        return out

    def frac(x):
        return round(x / PEAK_BF16_TFLOPS, 4)

    W = workload(args.workload, args.window, args.attn_chunk)
    wl, prob, bufs = W["wl"], W["prob"], W["bufs"]

    if args.kernels_only:
        W["gathers"]()
        for r in wl.ranks:
            W["fwd"](r)
        launches = chunk_launches(api, prob, wl, W["k_ring"], W["v_ring"])
        kr = kernel_rates(api, ctx, prob, wl, bufs, launches, compute, wl.backward, reps=1)
        # the calibration copies of the traffic record: the layout gather of K and one staging copy
        api.ra_layout_gather(ctx, prob, 0, wl.cp, W["dev"]["k"], W["k_ring"])
        api.ra_stage_kv(ctx, prob, 0, W["k_ring"], W["v_ring"])
        torch.cuda.synchronize()
        print(json.dumps({"kernels_only": wl.name, "kernels": kr}), flush=True)
        ctx.close()
        return

    # ---- the headline: whole steps of the workload, median step time
    R = rates(W, args.steps, args.warmup)
    value = R["tflops"]

    # ---- each chunk kernel on its own (event-timed replays of the workload's launches)
    launches = chunk_launches(api, prob, wl, W["k_ring"], W["v_ring"])
    kr = kernel_rates(api, ctx, prob, wl, bufs, launches, compute, wl.backward)
    del launches
    dom = max(kr, key=lambda k: kr[k]["total_ms_per_pass"])
    d = kr[dom]
    traffic = stored_traffic(wl.name, dom)
    roof = {"kernel": dom, "bound": "mfma", "achieved": d["achieved_tflops"], "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": d["frac"],
            "traffic": None if traffic is None else round(traffic / 1e9 * 1e3) / 1e3,
            "traffic_unit": "GB per launch", "avg_launch_ms": d["avg_launch_ms"],
            "algorithmic_tflop_per_launch": d["algorithmic_tflop_per_launch"],
            "launches": d["launches"]}

    # ---- split-KV all-gather forward (the chunks computed concurrently into partials)
    ws_split = api.workspace(prob, 2)
    merge_stream = torch.cuda.Stream()

    def fwd_split():
        for r in wl.ranks:
            b = bufs[r]
            api.rank_view_fwd_split(ctx, prob, r, b["q"], W["k_ring"], W["v_ring"], ws=ws_split,
                                    compute=compute, merge=merge_stream, out=(b["o"], b["lse"]))
    split_ms, _ = timed_each(fwd_split, 3)
    del ws_split

    # ---- HBM-bound steps, cold (after writing a 2 GiB buffer, more than the 256 MB MALL and the
    # L2s hold) and warm (back to back)
    esize = 2 if wl.dtype == "bf16" else 4
    flush = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")

    def cold_warm(fn, nbytes, reps=5):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            flush.fill_(1)
            a.record(compute)
            fn()
            b.record(compute)
        torch.cuda.synchronize()
        cold = statistics.median(a.elapsed_time(b) for a, b in ev)
        warm, _ = timed_each(fn, reps)
        return {"bytes": nbytes, "cold_ms": round(cold, 4), "cold_gbs": round(nbytes / (cold * 1e-3) / 1e9, 1),
                "warm_ms": round(warm, 4), "warm_gbs": round(nbytes / (warm * 1e-3) / 1e9, 1)}

    hbm = {"peak_gbs": PEAK_HBM_GBS}
    kbytes = 2 * wl.batch * wl.heads_kv * wl.seq_len * wl.head_dim * esize
    hbm["layout_gather_k"] = cold_warm(lambda: api.ra_layout_gather(ctx, prob, 0, wl.cp, W["dev"]["k"], W["k_ring"]),
                                       kbytes)
    stage_dst = torch.empty((2, wl.batch, wl.heads_kv, prob.chunk, wl.head_dim), dtype=prob.torch_dtype,
                            device="cuda")
    sbytes = 2 * stage_dst.numel() * esize
    hbm["staging_copy"] = cold_warm(lambda: api.ra_stage_kv(ctx, prob, 1 % wl.cp, W["k_ring"], W["v_ring"], stage_dst),
                                    sbytes)
    del stage_dst
    U, m, l = api.new_state(prob, prob.chunk)
    api.ra_state_init(ctx, prob, U, m, l)
    o_part = torch.zeros_like(U)
    lse_part = torch.zeros_like(m)
    hbm["lse_merge"] = cold_warm(lambda: api.ra_lse_merge(ctx, prob, o_part, lse_part, U, m, l),
                                 wl.batch * wl.heads_q * prob.chunk * (12 * wl.head_dim + 20))
    del U, m, l, o_part, lse_part
    # Ulysses re-shard at the Qwen3-shaped share's source: 32 query heads over an all-to-all of
    # 8, full sequence 65536 (the receive buffer of one rank unpacked to its 4-head shard)
    uprob = api.Problem(1, 65536, 32, 8, 128, 8, "contiguous", "bf16")
    ushape = api.reshard_shapes(uprob, 1, 32)
    usrc = torch.zeros(ushape[0], dtype=torch.bfloat16, device="cuda")
    udst = torch.empty(ushape[1], dtype=torch.bfloat16, device="cuda")
    hbm["ulysses_reshard"] = cold_warm(lambda: api.ra_ulysses_reshard(ctx, uprob, 1, 32, usrc, udst),
                                       2 * usrc.numel() * 2)
    hbm["ulysses_reshard"]["shape"] = "head unpack, (8, 1, 4, 8192, 128) bf16 -> (1, 4, 65536, 128)"
    del usrc, udst, flush

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(R["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V/dO, bf16 round-to-nearest-even; model shapes only",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len,
                   "heads_q": wl.heads_q, "heads_kv": wl.heads_kv, "head_dim": wl.head_dim,
                   "cp": wl.cp, "layout": wl.layout, "ranks": list(wl.ranks),
                   "passes": "fwd+bwd" if wl.backward else "fwd",
                   "window": args.window, "attn_chunk": args.attn_chunk},
        "timing": "median over the timed steps of HIP events on the compute stream",
        "step_ms_all": R["step_ms_all"],
        "frac_of_peak": frac(value),
        "fwd_tflops": round(R["fwd_tflops"], 2), "fwd_frac_of_peak": frac(R["fwd_tflops"]),
        "counted_tflop_per_step": round(R["counted_tflop_per_step"], 4),
    }
    if wl.backward:
        out["bwd_tflops"] = round(R["bwd_tflops"], 2)
        out["bwd_frac_of_peak"] = frac(R["bwd_tflops"])
    out["split_kv_fwd"] = {"ms": round(split_ms, 4), "tflops": round(W["fwd_flops"] / (split_ms * 1e-3) / 1e12, 2),
                           "ring_fwd_ms": round(R["fwd_ms"], 4)}
    out["roofline"] = roof
    out["kernels"] = kr
    out["hbm_kernels"] = hbm
    if "chunk_fwd_pp_kernel" in kr:
        fk = kr["chunk_fwd_pp_kernel"]["total_ms_per_pass"]
        out["staging_overlap"] = {"rank_views_fwd_ms": round(R["fwd_ms"], 4), "chunk_kernels_fwd_ms": fk,
                                  "ratio": round(fk / R["fwd_ms"], 4)}
    if not args.no_cpu_baseline and args.workload == DEFAULT_WORKLOAD:
        out["cpu_baseline"] = cpu_baseline(wl, W["t"], args.cpu_seconds)
    del W, bufs, R
    torch.cuda.empty_cache()

    # ---- the other long-sequence workloads, rank views only
    if args.workload == DEFAULT_WORKLOAD and not args.no_extra:
        other = {}
        for name in EXTRA_WORKLOADS:
            W2 = workload(name)
            R2 = rates(W2, 3, 1)
            o = {"ms_per_step": round(R2["ms_per_step"], 4), "tflops": round(R2["tflops"], 2),
                 "frac_of_peak": frac(R2["tflops"]), "fwd_tflops": round(R2["fwd_tflops"], 2),
                 "fwd_frac_of_peak": frac(R2["fwd_tflops"])}
            if "bwd_tflops" in R2:
                o["bwd_tflops"] = round(R2["bwd_tflops"], 2)
                o["bwd_frac_of_peak"] = frac(R2["bwd_tflops"])
            other[name] = o
            del W2
            torch.cuda.empty_cache()
        out["other_workloads"] = other
    ctx.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
