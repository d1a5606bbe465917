#!/usr/bin/env python3
"""Benchmark of exact split-KV attention + merge on one MI355X.

One step = one fused ``splitkv_attn`` call (partial attention of every LPT unit,
then the log-sum-exp merge) over the whole workload, inputs resident in HBM.
Prints one JSON line. Default workload: 8 sequences with contexts in [4096, 32768],
16 trailing causal queries, GQA 32/8, head_dim 128, KV block 512, 256 workers (bf16).

    python bench.py [--steps K] [--warmup W] [--workload batch8|long|lognormal|mixed|decode|small]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "split-KV attention+merge effective HBM GB/s & TFLOP/s, % of MI355X roofline"


KERNEL_SOURCES = ("partial_bf16.hip", "partial_f32.hip", "merge.hip", "abi.cpp", "plan.cpp", "kernels.hpp",
                  "plan_image.hpp", "lds_tiles.hpp")


def _kernel_sha(csrc: str | None = None) -> str:
    """Hash of the forward path's sources with comments and blank space removed, so that
    an edit of comments alone does not mark the committed counter runs as stale."""
    csrc = csrc or os.path.join(ROOT, "split_kv_exact_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(wl_key: str):
    """HBM bytes per partial-attention launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources; otherwise None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{wl_key}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sha") != _kernel_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def _time_loop(fn, steps, stream, flush=None):
    """Mean milliseconds per call of fn over ``steps`` calls, timed with HIP events on
    the stream the library launches on. With ``flush``, each call is preceded (outside
    the events) by a write of a 1 GiB buffer that evicts L2 and the 256 MiB MALL."""
    import torch

    if flush is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        e1.synchronize()
        return e0.elapsed_time(e1) / steps
    tot = 0.0
    for _ in range(steps):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        tot += e0.elapsed_time(e1)
    return tot / steps


def _time_each(fn, steps, stream):
    """Mean milliseconds of fn, each call bracketed by its own pair of HIP events on
    the stream (kernel time without the gaps between back-to-back launches)."""
    import torch

    pairs = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        pairs.append((e0, e1))
    pairs[-1][1].synchronize()
    return sum(a.elapsed_time(b) for a, b in pairs) / steps


def cpu_baseline(wl, q, k, v, budget_s: float):
    """Time the oracle (float64, NumPy) on the host over (sequence, KV head) groups of
    the same workload, in order, until ``budget_s`` seconds of oracle work or the whole
    workload is done. Widening the device data to float64 is not timed."""

    from oracle import attend_rows
    from split_kv_exact_amd.metrics import visible_pairs  # noqa: F401
    from workloads import widen_to_f64

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    qo = np.concatenate([[0], np.cumsum(wl.q_lens)]).astype(np.int64)
    ko = np.concatenate([[0], np.cumsum(wl.kv_lens)]).astype(np.int64)
    g, d, es = wl.group, wl.head_dim, wl.elem_bytes
    sc = 1.0 / math.sqrt(d)
    spent, done_bytes, done_flops, groups = 0.0, 0, 0, 0
    total_groups = wl.batch * wl.num_kv_heads
    for s in range(wl.batch):
        n, qs = wl.kv_lens[s], wl.q_lens[s]
        for kap in range(wl.num_kv_heads):
            Qr = widen_to_f64(q[qo[s]:qo[s + 1], kap * g:(kap + 1) * g]).reshape(qs * g, d)
            Kh = widen_to_f64(k[ko[s]:ko[s + 1], kap])
            Vh = widen_to_f64(v[ko[s]:ko[s + 1], kap])
            pos = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)
            t0 = time.perf_counter()
            attend_rows(Qr, pos, Kh, Vh, sc, wl.causal)
            spent += time.perf_counter() - t0
            groups += 1
            done_bytes += qs * g * d * es + 2 * n * d * es + qs * g * (d + 1) * 4
            pairs = qs * n - qs * (qs - 1) // 2 if wl.causal else qs * n
            done_flops += 4 * d * g * pairs
            if spent >= budget_s:
                break
        if spent >= budget_s:
            break
    return {
        "value": round(done_bytes / spent / 1e9, 4),
        "unit": "GB/s",
        "tflops": round(done_flops / spent / 1e12, 6),
        "cores": int(threads),
        "kind": "oracle",
        "seconds": round(spent, 3),
        "sample": f"{groups} of {total_groups} (sequence, KV head) groups of the same workload, in order, "
                  f"float64 NumPy oracle (two-pass softmax by definition); effective bytes Q+K+V+O+LSE of "
                  f"the processed groups / oracle time",
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="batch8")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true", help="skip the cold-cache per-step measurement")
    ap.add_argument("--schedule", default="auto", choices=("auto", "queue", "static"),
                    help="how the partial-attention workgroups take their jobs (bf16)")
    ap.add_argument("--cost-ridge", type=int, default=0,
                    help="LPT unit cost: 0 = q * len * heads (the pages' cost); R > 0 = len * max(q * g, R) "
                         "per KV head (roofline-aware, R = ridge in query rows)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed fused steps for this long before the warmup steps (the GPU's clocks ramp up "
                         "over the first tens of milliseconds of work)")
    ap.add_argument("--no-xcd-calibration", action="store_true",
                    help="skip the calibration launches that measure the 8 XCDs' relative speeds and re-place "
                         "the plan's workers (most loaded on the fastest XCDs) before timing")
    ap.add_argument("--backward", action="store_true",
                    help="also time the backward pass (splitkv_attn_backward) and report it under 'backward'")
    ap.add_argument("--planner-study", action="store_true",
                    help="host only: time the LPT planner against an exact MILP balancer (HiGHS) on small "
                         "instances cut from the workloads, and on the full workloads, then exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (a kernel of known traffic, for scaling "
                         "hardware byte counters)")
    args = ap.parse_args()

    if args.planner_study:
        print(json.dumps(planner_study()), flush=True)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: split-KV here runs on the 256 CUs of a single MI355X; "
              "this benchmark has no multi-GPU mode (use --gpus 1).", file=sys.stderr)
        return 2

    import torch

    import split_kv_exact_amd as skv
    from split_kv_exact_amd import metrics as M
    from workloads import get_workload, make_qkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = get_workload(args.workload)
    print(f"[bench] workload {wl.name}: drawing inputs", file=sys.stderr, flush=True)
    q, k, v = make_qkv(wl, dev)

    # Planner (host) timing: median of repeated calls.
    plan_times = []
    for _ in range(20):
        t0 = time.perf_counter_ns()
        plan = skv.plan_for(wl, args.cost_ridge)
        plan_times.append((time.perf_counter_ns() - t0) / 1e6)
    plan_times.sort()
    info = plan.info()
    dev_plan = skv.splitkv_plan_upload(plan, dev)
    ws = skv.workspace(plan, dev)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()

    sched = args.schedule
    xcd_cal = None
    if not args.no_xcd_calibration and wl.num_workers % 8 == 0:
        print("[bench] XCD speed calibration", file=sys.stderr, flush=True)
        plan, dev_plan, xcd_cal = _calibrate_xcd(skv, wl, plan, dev_plan, q, k, v, ws, args.cost_ridge, dev)

    def step():
        skv.splitkv_attn(plan, dev_plan, q, k, v, ws, out, lse, schedule=sched)

    def partial():
        skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws, schedule=sched)

    def merge():
        skv.splitkv_merge(plan, dev_plan, ws, out, lse)

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    print("[bench] settle and warmup", file=sys.stderr, flush=True)
    settle_steps = 0
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_ms * 1e-3:
        for _ in range(4):
            step()
        settle_steps += 4
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly K fused steps, synchronised on both sides.
    print("[bench] timed steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ms_step = _time_loop(step, args.steps, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps

    # Dominant kernel (partial attention) and merge, each launched alone and timed per
    # launch: the kernel durations a kernel trace of this run reports.
    ms_partial = _time_each(partial, args.steps, stream)
    ms_merge = _time_each(merge, args.steps, stream)
    # Per-step spread: each fused step timed alone (median and minimum).
    per_step = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        per_step.append(e0.elapsed_time(e1))
    per_step.sort()
    # Measured per-CU time imbalance of one partial-attention launch: each workgroup's
    # start and end on the GPU's 100 MHz clock.
    clock = torch.zeros(2 * wl.num_workers, dtype=torch.int64, device=dev)
    skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws, schedule=sched, clock=clock)
    torch.cuda.synchronize()
    ck = clock.view(-1, 2).cpu().double()
    busy = (ck[:, 1] - ck[:, 0]) / 100.0  # microseconds
    measured = {
        "busy_us_mean": round(float(busy.mean()), 2),
        "busy_us_max": round(float(busy.max()), 2),
        "imbalance": round(float(busy.max() / busy.mean() - 1.0), 4),
        "end_spread_us": round(float((ck[:, 1].max() - ck[:, 1].min()) / 100.0), 2),
        # Workgroups are dealt to the 8 XCDs round-robin (workgroup w on XCD w % 8).
        "busy_us_mean_by_xcd": [round(float(busy[x::8].mean()), 1) for x in range(8)]
        if wl.num_workers % 8 == 0 else None,
    }
    ms_cold = None
    if not args.no_flush:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        ms_cold = _time_loop(step, max(3, min(args.steps, 10)), stream, flush)
        del flush
    torch.cuda.synchronize()

    eb, fl = M.effective_bytes(wl), M.flops(wl)
    gbs = eb / (ms_step * 1e-3) / 1e9
    tfs = fl / (ms_step * 1e-3) / 1e12
    bound = M.binding_roof(wl)
    pk_bytes = M.partial_kernel_bytes(wl)
    if bound == "hbm":
        achieved = pk_bytes / (ms_partial * 1e-3) / 1e9
        peak, unit = M.PEAK_HBM_GBS, "GB/s"
    else:
        achieved = fl / (ms_partial * 1e-3) / 1e12
        peak = M.PEAK_FP32_VECTOR_TFLOPS if wl.dtype == "float32" else M.PEAK_BF16_MFMA_TFLOPS
        unit = "TFLOP/s"
    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bfloat16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V drawn on the device)",
        "config": {"workload": wl.name, **{k_: v_ for k_, v_ in wl.summary().items() if k_ != "workload"}},
        "tflops": round(tfs, 3),
        "roofline_fraction_step": round(M.roofline_seconds(wl) / (ms_step * 1e-3), 4),
        "binding_roof": bound,
        "roofline": {
            "kernel": "partial attention (splitkv_partial_attn)",
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": _traffic(args.workload),
            "ms_per_launch": round(ms_partial, 5),
            "algorithmic_bytes_per_launch": pk_bytes,
        },
        "ms_per_step_median": round(per_step[len(per_step) // 2], 5),
        "ms_per_step_min": round(per_step[0], 5),
        "ms_merge_kernel": round(ms_merge, 5),
        "ms_per_step_cold_cache": None if ms_cold is None else round(ms_cold, 5),
        "wall_ms_per_step": round(wall_ms, 5),
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "effective_bytes": eb,
        "flops": fl,
        "lpt": {
            "units": info["num_units"],
            "workers": wl.num_workers,
            "cost_ridge_rows": args.cost_ridge,
            "imbalance": info["imbalance"],
            "makespan": info["makespan"],
            "lower_bound": info["lower_bound"],
            "plan_ms_median": round(plan_times[len(plan_times) // 2], 4),
            "schedule": sched,
            "xcd_calibration": xcd_cal,
            "measured_per_cu": measured,
        },
        "workspace_bytes": info["workspace_bytes"],
        "kernel_sha": _kernel_sha(),
    }
    if args.backward:
        result["backward"] = (_bench_backward(skv, M, wl, plan, dev_plan, q, k, v, ws, out, lse, stream, args)
                              if wl.dtype == "bfloat16" else None)  # the backward takes bf16 inputs
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


def _calibrate_xcd(skv, wl, plan, dev_plan, q, k, v, ws, ridge, dev, launches=5):
    """Relative speeds of the 8 XCDs from static launches of the plan: each workgroup's
    busy time on the GPU clock against its worker's planned load (workgroup w runs
    worker w and sits on XCD w % 8). Returns the plan rebuilt with those speeds (same
    units per worker, most loaded workers on the fastest XCDs), its device copy, and a
    summary."""
    import torch

    m = wl.num_workers
    load = plan.export()["load"].astype(np.float64)
    clock = torch.zeros(2 * m, dtype=torch.int64, device=dev)
    busy = np.zeros(m)
    for _ in range(launches):
        skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws, schedule="static", clock=clock)
        torch.cuda.synchronize()
        ck = clock.view(-1, 2).cpu().double().numpy()
        busy += ck[:, 1] - ck[:, 0]
    rate = np.array([load[x::8].sum() / max(busy[x::8].sum(), 1.0) for x in range(8)])
    speeds = [max(1, int(round(1000.0 * r / rate.max()))) for r in rate]
    plan2 = skv.plan_for(wl, ridge, speeds)
    dev_plan2 = skv.splitkv_plan_upload(plan2, dev)
    return plan2, dev_plan2, {
        "launches": launches,
        "busy_us_mean_by_xcd": [round(float(busy[x::8].mean()) / launches / 100.0, 1) for x in range(8)],
        "xcd_speed": speeds,
    }


def planner_study(milp_seconds: float = 20.0):
    """The Split-KV page ("Timeline") reports LPT planning three orders of magnitude
    faster than the best load-balancing baseline, which it does not name. Here the
    baseline is the exact one: the makespan MILP (x[u, w] binary, min C subject to
    every unit on one worker and every worker's load <= C), solved by HiGHS through
    SciPy with a time limit. Instances are the first sequences of the lognormal and
    mixed workloads with fewer heads and workers, so that the MILP stays small; the
    C++ planner's time on the full workloads is reported beside them."""
    from scipy.optimize import Bounds, LinearConstraint, milp

    import split_kv_exact_amd as skv
    from workloads import get_workload

    def c_plan(kv, ql, hq, hkv, b, m):
        times = []
        for _ in range(20):
            t0 = time.perf_counter_ns()
            pl = skv.splitkv_plan(kv, ql, hq, hkv, 128, b, m, True, 0)
            times.append((time.perf_counter_ns() - t0) / 1e3)
        times.sort()
        return pl, times[len(times) // 2]

    def exact(costs, m):
        n = len(costs)
        nv = n * m + 1
        obj = np.zeros(nv)
        obj[-1] = 1.0
        a1 = np.zeros((n, nv))
        a2 = np.zeros((m, nv))
        for u in range(n):
            a1[u, u * m:(u + 1) * m] = 1.0
        for w in range(m):
            a2[w, w:n * m:m] = costs
            a2[w, -1] = -1.0
        integ = np.ones(nv)
        integ[-1] = 0
        t0 = time.perf_counter()
        r = milp(obj, constraints=[LinearConstraint(a1, 1, 1), LinearConstraint(a2, -np.inf, 0)], integrality=integ,
                 bounds=Bounds(0, np.r_[np.ones(n * m), np.inf]), options={"time_limit": milp_seconds})
        return r, time.perf_counter() - t0

    rows = []
    for key, nseq, hq, hkv, b, m in (("lognormal", 2, 4, 1, 4096, 4), ("lognormal", 4, 4, 1, 4096, 8),
                                     ("mixed", 3, 8, 1, 4096, 8), ("mixed", 132, 8, 1, 65536, 16)):
        wl = get_workload(key)
        kv, ql = list(wl.kv_lens[:nseq]), list(wl.q_lens[:nseq])
        if key == "mixed" and nseq == 3:
            kv, ql = [kv[0], kv[1], wl.kv_lens[-1]], [ql[0], ql[1], wl.q_lens[-1]]  # two decode, one prefill
        pl, us = c_plan(kv, ql, hq, hkv, b, m)
        costs = pl.export()["unit_cost"].astype(np.float64)
        inf = pl.info()
        r, sec = exact(costs, m)
        rows.append({
            "instance": f"{key}: {len(kv)} sequences, Hq/Hkv {hq}/{hkv}, block {b}, {m} workers",
            "units": int(inf["num_units"]),
            "lpt_makespan": int(inf["makespan"]),
            "lower_bound": int(inf["lower_bound"]),
            "lpt_us": round(us, 1),
            "milp_makespan": None if r.x is None else int(round(r.fun)),
            "milp_proved_bound": None if getattr(r, "mip_dual_bound", None) is None else float(r.mip_dual_bound),
            "milp_optimal": bool(r.status == 0),
            "milp_s": round(sec, 2),
        })
    full = []
    for key in ("lognormal", "mixed", "batch8"):
        wl = get_workload(key)
        pl, us = c_plan(wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.block_len, wl.num_workers)
        inf = pl.info()
        full.append({"workload": wl.name, "units": int(inf["num_units"]), "workers": wl.num_workers,
                     "lpt_ms": round(us / 1e3, 3), "imbalance": inf["imbalance"],
                     "makespan_over_lower_bound": inf["makespan"] / inf["lower_bound"],
                     "milp_binaries": int(inf["num_units"]) * wl.num_workers})
    return {"study": "LPT planner against an exact makespan MILP (HiGHS via SciPy, "
                     f"{milp_seconds:.0f} s limit)", "instances": rows, "full_workloads": full}


def _bench_backward(skv, M, wl, plan, dev_plan, q, k, v, ws, out, lse, stream, args):
    """Times splitkv_attn_backward (its four launches together) at the forward's O and
    LSE, with a seeded upstream gradient."""
    import torch

    print("[bench] backward", file=sys.stderr, flush=True)
    gen = torch.Generator(device=q.device)
    gen.manual_seed(99)
    do = torch.randn(q.shape, generator=gen, device=q.device, dtype=torch.float32).to(q.dtype)
    skv.splitkv_attn(plan, dev_plan, q, k, v, ws, out, lse)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)

    def bstep():
        skv.splitkv_attn_backward(plan, dev_plan, q, k, v, do, out, lse, ws, dq, dk, dv)

    # Untimed calls while the clocks settle (as for the forward), then the warmups.
    t_settle = time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_ms * 1e-3:
        bstep()
        torch.cuda.synchronize()
    for _ in range(max(1, args.warmup)):
        bstep()
    ms = _time_loop(bstep, max(3, min(args.steps, 10)), stream)
    fl, by = M.backward_flops(wl), M.backward_bytes(wl)
    tr = M.backward_roofline_seconds(wl)
    bound = "mfma" if fl / (M.PEAK_BF16_MFMA_TFLOPS * 1e12) >= by / (M.PEAK_HBM_GBS * 1e9) else "hbm"
    return {
        "ms_per_call": round(ms, 5),
        "tflops": round(fl / (ms * 1e-3) / 1e12, 3),
        "gbs": round(by / (ms * 1e-3) / 1e9, 2),
        "flops": fl,
        "bytes": by,
        "bound": bound,
        "roofline_fraction": round(tr / (ms * 1e-3), 4),
        "note": "flops 10*D per visible (row, key) pair; bytes Q, K, V, dO, O, LSE read once, dQ, dK, dV written",
    }


if __name__ == "__main__":
    sys.exit(main())
