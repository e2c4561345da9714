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
DEFAULT_WORKLOAD = "llama-gqa-cp8-zigzag"


def counted_flops(api, prob, rank):
    """Forward FLOPs of one rank view by the metric's counting rule (per ring step)."""
    per_step = []
    for i in range(prob.cp):
        _, pairs = api.ra_plan_step(prob, rank, i)
        f = 0
        for q0, k0, ql, kl, mask in pairs:
            if mask == 0:
                f += 4 * prob.head_dim * ql * kl
            elif mask == 1:
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
    heads = list(range(n_rep))  # the query heads of key/value head 0
    q = t.as_f64("q")[:1, heads]
    k = t.as_f64("k")[:1, :1]
    v = t.as_f64("v")[:1, :1]
    do = t.as_f64("do")[:1, heads]
    kpos = np.arange(wl.seq_len)
    # take rows from the end of the slice (the rows with the most visible keys)

    def run(nrows):
        rows = pos[-nrows:]
        t0 = time.perf_counter()
        O.attention_rows(q[:, :, rows], k, v, rows, kpos)
        O.attention_rows_bwd(q[:, :, rows], k, v, do[:, :, rows], rows, kpos)
        dt = time.perf_counter() - t0
        vis = float(np.sum(rows + 1))  # keys visible to each row (causal, full sequence)
        flops = (4 + 10) * wl.head_dim * vis * len(heads)
        return dt, flops, rows

    n = 16
    dt, flops, rows = run(n)
    while dt < target_s / 8 and n < len(pos):
        n = min(len(pos), n * 4)
        dt, flops, rows = run(n)
    if dt < target_s / 2 and n < len(pos):
        n = min(len(pos), int(n * target_s / max(dt, 1e-3) * 0.8))
        dt, flops, rows = run(n)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"rank {rank} of {wl.name}: last {len(rows)} rows of the Q slice x {len(heads)} "
                      f"query heads (one key/value group), forward + backward over the full causal "
                      f"key prefix, FP64, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--same-stream", action="store_true", help="stage K/V on the compute stream")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build runs a single rank view at a time on one "
              "MI355X (the ring is simulated on one device); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    from context_blockwise_causal_amd import api
    from context_blockwise_causal_amd.inputs import draw
    from context_blockwise_causal_amd.workloads import WORKLOADS
    from tests.gpu_util import to_dev

    wl = WORKLOADS[args.workload]
    prob = api.Problem(wl.batch, wl.seq_len, wl.heads_q, wl.heads_kv, wl.head_dim, wl.cp,
                       wl.layout, wl.dtype)
    t = draw(wl.batch, wl.seq_len, wl.heads_q, wl.heads_kv, wl.head_dim, wl.dtype, wl.seed,
             with_grad=True)
    ctx = api.Context(0)
    dev = {n: to_dev(t.store[n], wl.dtype) for n in ("q", "k", "v", "do")}
    compute = torch.cuda.current_stream()
    staging = compute if args.same_stream else torch.cuda.Stream()

    # buffers allocated once, outside the timed region
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

    def step():
        api.ra_layout_gather(ctx, prob, 0, wl.cp, dev["k"], k_ring)
        api.ra_layout_gather(ctx, prob, 0, wl.cp, dev["v"], v_ring)
        for r in wl.ranks:
            api.ra_layout_gather(ctx, prob, r, 1, dev["q"], bufs[r]["q"])
            if wl.backward:
                api.ra_layout_gather(ctx, prob, r, 1, dev["do"], bufs[r]["do"])
            fwd(r)
            if wl.backward:
                bwd(r)

    def timed(fn, reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        torch.cuda.synchronize()
        ev[0].record(compute)
        for _ in range(reps):
            fn()
        ev[1].record(compute)
        torch.cuda.synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    fwd_flops = {r: sum(counted_flops(api, prob, r)) for r in wl.ranks}
    total_fwd = sum(fwd_flops.values())
    total = total_fwd * (3.5 if wl.backward else 1.0)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    step_ms = timed(step, args.steps)

    # per-pass rates, timed separately (same launches as inside the step)
    fwd_ms = timed(lambda: [fwd(r) for r in wl.ranks], max(2, args.steps))
    bwd_ms = timed(lambda: [bwd(r) for r in wl.ranks], max(2, args.steps)) if wl.backward else None

    # dominant kernel: replay the chunk launches of the first rank view with events on the
    # launch stream, to get the kernel's own average duration.
    roof = kernel_roofline(api, ctx, prob, wl, dev, k_ring, v_ring, bufs, compute, wl.backward)

    value = total / (step_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.dtype,
        "data": "synthetic: seeded N(0,1) Q/K/V/dO, bf16 round-to-nearest-even; model shapes only",
        "config": {"workload": wl.name, "batch": wl.batch, "seq_len": wl.seq_len,
                   "heads_q": wl.heads_q, "heads_kv": wl.heads_kv, "head_dim": wl.head_dim,
                   "cp": wl.cp, "layout": wl.layout, "ranks": list(wl.ranks),
                   "passes": "fwd+bwd" if wl.backward else "fwd"},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "fwd_tflops": round(total_fwd / (fwd_ms * 1e-3) / 1e12, 2),
        "fwd_frac_of_peak": round(total_fwd / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "counted_tflop_per_step": round(total / 1e12, 4),
    }
    if wl.backward:
        bt = total_fwd * 2.5 / (bwd_ms * 1e-3) / 1e12
        out["bwd_tflops"] = round(bt, 2)
        out["bwd_frac_of_peak"] = round(bt / PEAK_BF16_TFLOPS, 4)
    out["roofline"] = roof
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl, t, args.cpu_seconds)
    ctx.close()
    print(json.dumps(out), flush=True)


def kernel_roofline(api, ctx, prob, wl, dev, k_ring, v_ring, bufs, stream, backward):
    import torch
    r = wl.ranks[0]
    b = bufs[r]
    chunk = prob.chunk
    launches = []
    for i in range(prob.cp):
        owner, pairs = api.ra_plan_step(prob, r, i)
        if all(p[4] == 2 for p in pairs):
            continue
        f = counted_flops(api, prob, r)[i] * (2.5 if backward else 1.0)
        kc = k_ring[:, :, owner * chunk:(owner + 1) * chunk].contiguous()
        vc = v_ring[:, :, owner * chunk:(owner + 1) * chunk].contiguous()
        launches.append((pairs, kc, vc, f))
    if backward:
        name = "chunk_bwd_bf16_kernel"
        delta = api.ra_bwd_preprocess(ctx, prob, b["o"], b["do"])
        dq = torch.zeros((prob.batch, prob.heads_q, chunk, prob.head_dim), device="cuda")
        dk = torch.zeros((prob.batch, prob.heads_kv, chunk, prob.head_dim), device="cuda")
        dv = torch.zeros_like(dk)
        run = lambda L: api.ra_chunk_bwd(ctx, prob, b["q"], b["do"], b["lse"], delta, L[1], L[2], L[0],
                                         dq, dk, dv, stream)
    else:
        name = "chunk_fwd_bf16_kernel"
        U, m, l = api.new_state(prob, chunk)
        api.ra_state_init(ctx, prob, U, m, l)
        run = lambda L: api.ra_chunk_fwd(ctx, prob, b["q"], L[1], L[2], L[0], U, m, l, stream)
    for L in launches:
        run(L)
    torch.cuda.synchronize()
    reps = 3
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]
    times = [0.0] * len(launches)
    for _ in range(reps):
        for j, L in enumerate(launches):
            ev[j][0].record(stream)
            run(L)
            ev[j][1].record(stream)
        torch.cuda.synchronize()
        for j in range(len(launches)):
            times[j] += ev[j][0].elapsed_time(ev[j][1]) / reps
    flops = sum(L[3] for L in launches)
    avg_ms = sum(times) / len(launches)
    achieved = flops / len(launches) / (avg_ms * 1e-3) / 1e12
    return {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None, "avg_launch_ms": round(avg_ms, 4), "launches_per_rank_view": len(launches),
            "rank": r, "per_launch_ms": [round(x, 4) for x in times]}


if __name__ == "__main__":
    main()
