#!/usr/bin/env python3
"""Benchmark of exact split-KV attention + merge on one MI355X.

One step = one fused ``splitkv_attn`` call (partial attention of every LPT unit,
then the log-sum-exp merge) over the whole workload, inputs resident in HBM.
Prints one JSON line. Default workload: the largest one that fits one GPU, the mixed
batch of 128 decode sequences (1 query, contexts 8K-128K) and 4 prefill chunks (2048
queries over 64K contexts), GQA 64/8, head_dim 128, KV block 8192, 256 workers (bf16);
the decode-only part of that batch and the 8-sequence batch (the memory-bound shapes)
are timed after it and reported under "sub_runs". Every timed step starts from cold
caches (a 1 GiB write before it, outside its events).

    python bench.py [--steps K] [--warmup W] [--workload mixed|batch8|long|lognormal|decode|small]
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


KERNEL_SOURCES = ("partial_bf16.hip", "partial_mma.hip", "partial_f32.hip", "abi.cpp", "plan.cpp",
                  "kernels.hpp", "plan_image.hpp", "lds_tiles.hpp")


def _kernel_sha(csrc: str | None = None) -> str:
    """Hash of the partial-attention launch's sources (the kernels, the plan and the
    launch code; the merge is a separate kernel) with comments and blank space removed,
    so that an edit of comments alone does not mark the committed counter runs as stale."""
    csrc = csrc or os.path.join(ROOT, "split_kv_exact_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _traffic(wl_key: str, wl_name: str):
    """HBM bytes per partial-attention launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources and on this workload (its name holds
    its shape and block size); otherwise None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{wl_key}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        t = json.load(f)
    if t.get("kernel_sha") != _kernel_sha() or t.get("workload") != wl_name:
        return None
    return t.get("hbm_bytes_per_launch")


def _time_loop(fn, steps, stream):
    """Mean milliseconds per call of fn over ``steps`` back-to-back calls (warm caches),
    timed with HIP events on the stream the library launches on."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / steps


def _time_flushed(fn, steps, stream, flush):
    """Milliseconds of each of ``steps`` calls of fn, each bracketed by its own HIP events
    on the library's stream and preceded, outside the events, by a write of ``flush`` (1
    GiB), which evicts L2 and the 256 MiB MALL: every call starts from cold caches."""
    import torch

    times = []
    for _ in range(steps):
        flush.fill_(1.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    return times


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


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_threads() -> tuple:
    """(CPUs this process may run on, threads the oracle's BLAS is given): the affinity
    set, capped by OMP_NUM_THREADS where the environment sets it."""
    avail = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    cap = int(env) if env.isdigit() and int(env) > 0 else avail
    return avail, max(1, min(avail, cap))


def cpu_baseline(wl, q, k, v, budget_s: float, full: bool = False):
    """Time the oracle (float64, NumPy) on the host over (sequence, KV head) groups of the
    same workload. With ``full`` every group is timed. Otherwise groups are taken from
    two strata (at most 64 query rows per KV head, i.e. streaming-bound, and more rows),
    alternately and in a seeded random order within each, until ``budget_s`` seconds of
    oracle work; the full-workload time is then estimated per stratum (mean time of a
    sampled group times the stratum's group count). Widening device data to float64 is
    not timed."""
    from oracle import attend_rows
    from workloads import widen_to_f64

    avail, threads = _cpu_threads()
    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(limits=threads, user_api="blas")
    except Exception:
        limiter = None
    qo = np.concatenate([[0], np.cumsum(wl.q_lens)]).astype(np.int64)
    ko = np.concatenate([[0], np.cumsum(wl.kv_lens)]).astype(np.int64)
    g, d, es = wl.group, wl.head_dim, wl.elem_bytes
    sc = 1.0 / math.sqrt(d)
    groups = [(s, kap) for s in range(wl.batch) for kap in range(wl.num_kv_heads)]
    strata = [[x for x in groups if wl.q_lens[x[0]] * g <= 64], [x for x in groups if wl.q_lens[x[0]] * g > 64]]
    rng = np.random.default_rng(2024)
    order = []
    queues = [list(np.array(st, dtype=np.int64)[rng.permutation(len(st))]) if st else [] for st in strata]
    while any(queues):
        for qu in queues:
            if qu:
                order.append(tuple(int(x) for x in qu.pop(0)))
    spent = 0.0
    t_by = [[], []]
    done_bytes = 0
    try:
        for s, kap in order:
            n, qs = wl.kv_lens[s], wl.q_lens[s]
            Qr = widen_to_f64(q[qo[s]:qo[s + 1], kap * g:(kap + 1) * g]).reshape(qs * g, d)
            Kh = widen_to_f64(k[ko[s]:ko[s + 1], kap])
            Vh = widen_to_f64(v[ko[s]:ko[s + 1], kap])
            pos = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)
            t0 = time.perf_counter()
            attend_rows(Qr, pos, Kh, Vh, sc, wl.causal)
            dt = time.perf_counter() - t0
            spent += dt
            t_by[0 if qs * g <= 64 else 1].append(dt)
            done_bytes += qs * g * d * es + 2 * n * d * es + qs * g * (d + 1) * 4
            # Stop at the budget once every stratum holds a timed group.
            if not full and spent >= budget_s and all(t or not st for t, st in zip(t_by, strata)):
                break
    finally:
        if limiter is not None:
            limiter.unregister()
    ndone = sum(len(t) for t in t_by)
    complete = ndone == len(groups)
    est = spent if complete else sum(np.mean(t) * len(st) for t, st in zip(t_by, strata) if t)
    from split_kv_exact_amd.metrics import effective_bytes, flops

    eb, fl = effective_bytes(wl), flops(wl)
    return {
        "value": round(eb / est / 1e9, 4),
        "unit": "GB/s",
        "tflops": round(fl / est / 1e12, 6),
        "cores": int(threads),
        "cores_available": int(avail),
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "complete": bool(complete),
        "groups_timed": int(ndone),
        "groups_total": len(groups),
        "seconds_timed": round(spent, 3),
        "seconds_full_workload": round(est, 3),
        "sample_rate_gbs": round(done_bytes / spent / 1e9, 4),
        "sample": (f"{ndone} of {len(groups)} (sequence, KV head) groups of the same workload"
                   + (" (all)" if complete else
                      f", taken alternately from the streaming-bound (<= 64 rows per KV head: "
                      f"{len(t_by[0])} of {len(strata[0])}) and compute-bound ({len(t_by[1])} of "
                      f"{len(strata[1])}) strata in seeded random order; value = effective bytes of the whole "
                      f"workload / its estimated oracle time (mean time per sampled group x groups, per stratum)")
                   + f"; float64 NumPy oracle (two-pass softmax by definition), BLAS on {threads} threads, "
                     f"elementwise NumPy on one"),
    }


def measure(skv, M, wl, q, k, v, args, dev, stream, xcd=True, flush=None):
    """Everything the JSON line reports for one workload: the plan, XCD calibration,
    settled clocks, the timed fused steps (cold caches unless no flush buffer is given),
    the partial-attention and merge kernels per launch, and the measured per-CU busy time."""
    import torch

    plan_times = []
    for _ in range(20):
        t0 = time.perf_counter_ns()
        plan = skv.plan_for(wl, args.cost_ridge)
        plan_times.append((time.perf_counter_ns() - t0) / 1e6)
    plan_times.sort()
    info = plan.info()
    torch.cuda.synchronize()
    t0 = time.perf_counter_ns()
    dev_plan = skv.splitkv_plan_upload(plan, dev)
    torch.cuda.synchronize()
    upload_ms = (time.perf_counter_ns() - t0) / 1e6
    ws = skv.workspace(plan, dev)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device=dev)
    sched = args.schedule
    xcd_cal = None
    if xcd and not args.no_xcd_calibration and wl.num_workers % 8 == 0:
        print(f"[bench] {wl.name}: XCD speed calibration", file=sys.stderr, flush=True)
        plan, dev_plan, xcd_cal = _calibrate_xcd(skv, wl, plan, dev_plan, q, k, v, ws, args.cost_ridge, dev)

    def step():
        skv.splitkv_attn(plan, dev_plan, q, k, v, ws, out, lse, schedule=sched)

    def partial():
        skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws, schedule=sched)

    def merge():
        skv.splitkv_merge(plan, dev_plan, ws, out, lse)

    print(f"[bench] {wl.name}: settle and warmup", file=sys.stderr, flush=True)
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

    # Timed region: exactly K fused steps, synchronised on both sides; each one from
    # cold caches (flush outside its events) unless no flush buffer is given.
    print(f"[bench] {wl.name}: timed steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    if flush is not None:
        per_step = _time_flushed(step, args.steps, stream, flush)
    else:
        per_step = []
        for _ in range(args.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            e1.synchronize()
            per_step.append(e0.elapsed_time(e1))
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    ms_step = sum(per_step) / len(per_step)
    srt = sorted(per_step)
    # Back-to-back steps with warm caches, for comparison.
    ms_warm = _time_loop(step, args.steps, stream)
    # Dominant kernel (partial attention) and merge, each launched alone and timed per
    # launch: the kernel durations a kernel trace of this run reports.
    ms_partial = _time_each(partial, args.steps, stream)
    ms_merge = _time_each(merge, args.steps, stream)
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
    exec_info = plan.info()
    del ws, out, lse
    eb, fl = M.effective_bytes(wl), M.flops(wl)
    bound = M.binding_roof(wl)
    if bound == "hbm":
        achieved = eb / (ms_partial * 1e-3) / 1e9
        peak, unit = M.PEAK_HBM_GBS, "GB/s"
    else:
        achieved = fl / (ms_partial * 1e-3) / 1e12
        peak, unit = M.peak_flops_tflops(wl), "TFLOP/s"
    auto_q = exec_info["auto_schedule"] == 1
    ran = sched if sched != "auto" else ("queue" if auto_q else "static")
    return {
        "ms_per_step": ms_step,
        "ms_per_step_median": srt[len(srt) // 2],
        "ms_per_step_min": srt[0],
        "ms_per_step_warm": ms_warm,
        "cold_cache": flush is not None,
        "wall_ms_per_step": wall_ms,
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "gbs": eb / (ms_step * 1e-3) / 1e9,
        "tflops": fl / (ms_step * 1e-3) / 1e12,
        "roofline_fraction_step": M.roofline_seconds(wl) / (ms_step * 1e-3),
        "bound": bound,
        "roofline": {
            "kernel": "partial attention (splitkv_partial_attn)",
            "bound": bound,
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": _traffic(_wl_key(wl), wl.name),
            "ms_per_launch": round(ms_partial, 5),
            "algorithmic_bytes_per_launch": eb,
            "algorithmic_flops_per_launch": fl,
            "partial_workspace_bytes_uncredited": M.partial_traffic_bytes(wl),
        },
        "ms_merge_kernel": round(ms_merge, 5),
        "effective_bytes": eb,
        "flops": fl,
        "lpt": {
            "units": info["num_units"],
            "jobs": exec_info["num_jobs"],
            "workers": wl.num_workers,
            "cost_ridge_rows": args.cost_ridge,
            "imbalance": info["imbalance"],
            "makespan": info["makespan"],
            "lower_bound": info["lower_bound"],
            "plan_ms_median": round(plan_times[len(plan_times) // 2], 4),
            "plan_upload_ms": round(upload_ms, 4),
            "plan_bytes": int(info["plan_bytes"]),
            "schedule": sched,
            "schedule_run": ran,
            "executed": {
                "static_lists_page_cost": round(exec_info["exec_imbalance_static"], 6),
                "static_lists_job_estimate": round(exec_info["exec_imbalance_static_est"], 6),
                "queue_simulated_job_estimate": round(exec_info["exec_imbalance_queue_est"], 6),
            },
            "xcd_calibration": xcd_cal,
            "measured_per_cu": measured,
        },
        "workspace_bytes": info["workspace_bytes"],
    }


_WL_KEYS = {}


def _wl_key(wl) -> str:
    return _WL_KEYS.get(wl.name, wl.name)


def _r(x, n=5):
    return round(float(x), n)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixed")
    ap.add_argument("--sub-runs", default="auto",
                    help="comma-separated workloads timed after the main one and reported under 'sub_runs' "
                         "('auto': the decode-only sub-run and batch8 when the main workload is mixed; 'none')")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--cpu-full", action="store_true", help="time the oracle over the whole workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flush", action="store_true",
                    help="time the steps back to back from warm caches instead of after a 1 GiB flush each")
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
                    help="time the backward pass (splitkv_attn_backward) and report it under 'backward' "
                         "(the default for bf16 workloads; kept for explicit use)")
    ap.add_argument("--no-backward", action="store_true", help="do not time the backward pass")
    ap.add_argument("--planner-study", action="store_true",
                    help="host only: time the LPT planner against an exact MILP balancer (HiGHS) and write "
                         "the study as JSON, then exit")
    ap.add_argument("--planner-study-out", default=None, help="file for the planner study's JSON")
    ap.add_argument("--planner-study-quick", action="store_true", help="small instances only (for tests)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 1 GiB device copy (a kernel of known traffic, for scaling "
                         "hardware byte counters)")
    args = ap.parse_args()

    if args.planner_study:
        res = planner_study(quick=args.planner_study_quick)
        text = json.dumps(res, indent=1)
        if args.planner_study_out:
            with open(args.planner_study_out, "w") as f:
                f.write(text + "\n")
        print(json.dumps(res), flush=True)
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
    _WL_KEYS[wl.name] = args.workload
    print(f"[bench] workload {wl.name}: drawing inputs", file=sys.stderr, flush=True)
    q, k, v = make_qkv(wl, dev)
    stream = torch.cuda.current_stream()
    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # reads 1 GiB, writes 1 GiB
        torch.cuda.synchronize()
        del src, dst
    flush = None if args.no_flush else torch.empty(1 << 28, dtype=torch.float32, device=dev)
    r = measure(skv, M, wl, q, k, v, args, dev, stream, flush=flush)

    result = {
        "metric": METRIC,
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": _r(r["ms_per_step"]),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bfloat16" else "f32",
        "data": "synthetic (seeded N(0,1) Q/K/V drawn on the device)",
        "config": {"workload": wl.name, **{k_: v_ for k_, v_ in wl.summary().items() if k_ != "workload"}},
        "tflops": round(r["tflops"], 3),
        "roofline_fraction_step": round(r["roofline_fraction_step"], 4),
        "binding_roof": r["bound"],
        "roofline": r["roofline"],
        "ms_per_step_median": _r(r["ms_per_step_median"]),
        "ms_per_step_min": _r(r["ms_per_step_min"]),
        "cold_cache": r["cold_cache"],
        "ms_per_step_warm": _r(r["ms_per_step_warm"]),
        "ms_merge_kernel": r["ms_merge_kernel"],
        "wall_ms_per_step": _r(r["wall_ms_per_step"]),
        "settle": r["settle"],
        "effective_bytes": r["effective_bytes"],
        "flops": r["flops"],
        "lpt": r["lpt"],
        "workspace_bytes": r["workspace_bytes"],
        "kernel_sha": _kernel_sha(),
    }

    subs = args.sub_runs
    if subs == "auto":
        subs = "decode,batch8" if args.workload == "mixed" else "none"
    sub_out = {}
    for key in [x for x in subs.split(",") if x and x != "none"]:
        swl = get_workload(key)
        _WL_KEYS[swl.name] = key
        if args.workload == "mixed" and key == "decode":
            # The decode sequences are the mixed batch's first 128: their slices of its
            # tensors (same lengths, same recipe, packed by sequence).
            sq, sk, sv = q[:swl.total_q], k[:swl.total_kv], v[:swl.total_kv]
            src = "the mixed batch's tensors, its 128 decode sequences"
        else:
            sq, sk, sv = make_qkv(swl, dev)
            src = "own seeded draw"
        sr = measure(skv, M, swl, sq, sk, sv, args, dev, stream, flush=flush)
        rf = sr["roofline"]
        sub_out[key] = {
            "workload": swl.name,
            "inputs": src,
            "ms_per_step": _r(sr["ms_per_step"]),
            "ms_per_step_median": _r(sr["ms_per_step_median"]),
            "ms_per_step_min": _r(sr["ms_per_step_min"]),
            "ms_per_step_warm": _r(sr["ms_per_step_warm"]),
            "value": round(sr["gbs"], 2),
            "unit": "GB/s",
            "tflops": round(sr["tflops"], 3),
            "roofline_fraction_step": round(sr["roofline_fraction_step"], 4),
            "hbm_fraction_step": round(sr["gbs"] / M.PEAK_HBM_GBS, 4),
            "target_70pct_hbm_met": bool(sr["bound"] == "hbm" and sr["gbs"] >= 0.7 * M.PEAK_HBM_GBS),
            "roofline": rf,
            "ms_merge_kernel": sr["ms_merge_kernel"],
            "lpt": sr["lpt"],
        }
        del sq, sk, sv
    if sub_out:
        result["sub_runs"] = sub_out
    if flush is not None:
        del flush
    if not args.no_backward:
        result["backward"] = (_bench_backward(skv, M, wl, q, k, v, stream, args)
                              if wl.dtype == "bfloat16" else None)  # the backward takes bf16 inputs
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, args.cpu_budget, args.cpu_full)
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


def milp_makespan(costs, m, time_limit, aggregate=False):
    """The exact makespan balancer: min C subject to every unit on exactly one of m
    identical workers and every worker's load <= C, solved by HiGHS (SciPy). With
    ``aggregate`` the units of equal cost are one class and the integer variable
    y[c, w] counts the class-c units on worker w (the same optimum: equal-cost units are
    interchangeable), which keeps workload-sized instances to (classes x workers)
    variables. (Ordering the workers' loads to break their symmetry is valid too, but
    then HiGHS found no feasible point within a minute on the whole workloads.) Returns
    (result, seconds, variables)."""
    from scipy.optimize import Bounds, LinearConstraint, milp

    costs = np.asarray(costs, dtype=np.float64)
    if aggregate:
        cls, cnt = np.unique(costs, return_counts=True)
    else:
        cls, cnt = costs, np.ones(len(costs))
    nc = len(cls)
    nv = nc * m + 1
    obj = np.zeros(nv)
    obj[-1] = 1.0
    a1 = np.zeros((nc, nv))
    for c in range(nc):
        a1[c, c * m:(c + 1) * m] = 1.0
    a2 = np.zeros((m, nv))
    for w in range(m):
        a2[w, w:nc * m:m] = cls
        a2[w, -1] = -1.0
    cons = [LinearConstraint(a1, cnt, cnt), LinearConstraint(a2, -np.inf, 0)]
    ub = np.r_[np.repeat(cnt, m), np.inf]
    integ = np.ones(nv)
    integ[-1] = 0
    t0 = time.perf_counter()
    r = milp(obj, constraints=cons, integrality=integ, bounds=Bounds(0, ub),
             options={"time_limit": float(time_limit), "disp": False, "mip_rel_gap": 0.0})
    return r, time.perf_counter() - t0, nv


def planner_study(milp_seconds: float = 20.0, full_seconds: float = 60.0, quick: bool = False):
    """The Split-KV page ("Timeline") reports LPT planning three orders of magnitude
    faster than the best load-balancing baseline, which it does not name. Here the
    baseline is the exact one, the makespan MILP solved by HiGHS through SciPy with a
    time limit: per unit on small instances cut from the workloads (first sequences,
    fewer heads and workers), and aggregated by cost class on the full workloads (13k-19k
    units on 256 workers). Against each, the C++ planner's time (median of 20 calls), its
    makespan, and where the MILP proves one, the optimum or the solver's lower bound and
    the remaining gap. ``quick`` keeps the small instances only, with a short limit."""
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

    def row(name, kv, ql, hq, hkv, b, m, limit, aggregate):
        pl, us = c_plan(kv, ql, hq, hkv, b, m)
        costs = pl.export()["unit_cost"]
        inf = pl.info()
        r, sec, nv = milp_makespan(costs, m, limit, aggregate)
        found = r.x is not None
        bound = getattr(r, "mip_dual_bound", None)
        bound = None if bound is None or not np.isfinite(bound) else float(bound)
        lb_trivial = int(inf["lower_bound"])
        best_lb = max(lb_trivial, math.ceil(bound - 1e-6) if bound is not None else 0)
        return {
            "instance": name,
            "units": int(inf["num_units"]),
            "workers": m,
            "cost_classes": int(len(np.unique(costs))),
            "milp_formulation": "aggregated by cost class" if aggregate else "one binary per (unit, worker)",
            "milp_variables": int(nv),
            "lpt_makespan": int(inf["makespan"]),
            "lpt_us": round(us, 1),
            "lpt_imbalance": inf["imbalance"],
            "trivial_lower_bound": lb_trivial,
            "milp_status": int(r.status),
            "milp_optimal": bool(r.status == 0),
            "milp_makespan": int(round(r.fun)) if found else None,
            "milp_lower_bound": bound,
            "lpt_over_best_lower_bound": int(inf["makespan"]) / best_lb,
            "milp_s": round(sec, 2),
            "milp_time_limit_s": limit,
            "time_ratio_milp_over_lpt": round(sec / (us * 1e-6), 1),
        }

    rows = []
    small = (("lognormal", 2, 4, 1, 4096, 4), ("lognormal", 4, 4, 1, 4096, 8), ("mixed", 3, 8, 1, 4096, 8),
             ("mixed", 132, 8, 1, 65536, 16))
    for key, nseq, hq, hkv, b, m in small[:3] if quick else small:
        wl = get_workload(key)
        kv, ql = list(wl.kv_lens[:nseq]), list(wl.q_lens[:nseq])
        if key == "mixed" and nseq == 3:
            kv, ql = [kv[0], kv[1], wl.kv_lens[-1]], [ql[0], ql[1], wl.q_lens[-1]]  # two decode, one prefill
        name = f"{key}: {len(kv)} sequences, Hq/Hkv {hq}/{hkv}, block {b}, {m} workers"
        rows.append(row(name, kv, ql, hq, hkv, b, m, 5.0 if quick else milp_seconds, False))
    full = []
    if not quick:
        for key in ("lognormal", "mixed", "decode", "batch8"):
            wl = get_workload(key)
            full.append(row(f"{key}: the whole workload ({wl.name})", wl.kv_lens, wl.q_lens, wl.num_q_heads,
                            wl.num_kv_heads, wl.block_len, wl.num_workers, full_seconds, True))
    return {"study": "LPT planner against the exact makespan MILP (HiGHS via SciPy); small instances per unit, "
                     "whole workloads aggregated by cost class",
            "cpu_model": _cpu_model(), "instances": rows, "full_workloads": full}


def _bench_backward(skv, M, wl, q, k, v, stream, args):
    """Times splitkv_attn_backward (all its launches together) at the forward's O and
    LSE, with a seeded upstream gradient, once with fp32 and once with bf16 dK and dV.
    Mean of back-to-back calls after the same settling as the forward; not part of the
    headline value."""
    import torch

    print("[bench] backward", file=sys.stderr, flush=True)
    plan = skv.plan_for(wl, args.cost_ridge)
    dev_plan = skv.splitkv_plan_upload(plan, q.device)
    ws = skv.workspace(plan, q.device)
    gen = torch.Generator(device=q.device)
    gen.manual_seed(99)
    do = torch.randn(q.shape, generator=gen, device=q.device, dtype=torch.float32).to(q.dtype)
    out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v, ws)
    dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    res = {}
    # dK and dV as fp32, then as bf16 (the input dtype); dQ is fp32 in both.
    for dt, key in ((torch.float32, "fp32_dkv"), (torch.bfloat16, "bf16_dkv")):
        dk = torch.empty(k.shape, dtype=dt, device=q.device)
        dv = torch.empty(v.shape, dtype=dt, device=q.device)

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
        dkv_bytes = dk.element_size()
        fl, by = M.backward_flops(wl), M.backward_bytes(wl, dkv_bytes)
        tr = M.backward_roofline_seconds(wl, dkv_bytes)
        bound = "mfma" if fl / (M.PEAK_BF16_MFMA_TFLOPS * 1e12) >= by / (M.PEAK_HBM_GBS * 1e9) else "hbm"
        res[key] = {
            "ms_per_call": round(ms, 5),
            "tflops": round(fl / (ms * 1e-3) / 1e12, 3),
            "gbs": round(by / (ms * 1e-3) / 1e9, 2),
            "flops": fl,
            "bytes": by,
            "bound": bound,
            "roofline_fraction": round(tr / (ms * 1e-3), 4),
        }
        del dk, dv
    res["note"] = ("flops 10*D per visible (row, key) pair; bytes Q, K, V, dO, O, LSE read once, dQ (fp32), "
                   "dK, dV (fp32 or bf16) written")
    return res


if __name__ == "__main__":
    sys.exit(main())
