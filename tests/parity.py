"""Helpers for GPU-vs-oracle parity tests: run the library, widen results, compare.

Tolerances: fp32 inputs, output max|diff| <= 1e-5; bf16 inputs, output max|diff| <=
1e-2 and relative L2 <= 5e-3; log-sum-exp max|diff| <= 1e-4 in both; -inf must match
exactly (partials of rows that see no key of a block).
"""

from __future__ import annotations

import math
import sys
from dataclasses import dataclass

import numpy as np

TOL = {
    "float32": dict(o_max=1e-5, o_rel=None, lse=1e-4),
    "bfloat16": dict(o_max=1e-2, o_rel=5e-3, lse=1e-4),
}


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class Diff:
    o_max: float
    o_rel: float
    lse_max: float

    def __str__(self):
        return f"max|dO|={self.o_max:.3e} relL2={self.o_rel:.3e} max|dLSE|={self.lse_max:.3e}"


def compare(o_got, o_ref, l_got, l_ref) -> Diff:
    o_got = np.asarray(o_got, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    l_got = np.asarray(l_got, np.float64)
    l_ref = np.asarray(l_ref, np.float64)
    assert np.all(np.isfinite(o_got)), "non-finite output"
    assert not np.any(np.isnan(l_got)), "NaN log-sum-exp"
    ninf_ref = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l_got), ninf_ref), "-inf pattern of LSE differs"
    fin = ~ninf_ref
    lse_max = float(np.max(np.abs(l_got[fin] - l_ref[fin]))) if fin.any() else 0.0
    d = o_got - o_ref
    o_max = float(np.max(np.abs(d))) if d.size else 0.0
    nref = float(np.linalg.norm(o_ref))
    o_rel = float(np.linalg.norm(d) / nref) if nref > 0 else float(np.linalg.norm(d))
    return Diff(o_max, o_rel, lse_max)


def assert_within(diff: Diff, dtype: str, what: str) -> None:
    t = TOL[dtype]
    assert diff.o_max <= t["o_max"], f"{what}: {diff}"
    if t["o_rel"] is not None:
        assert diff.o_rel <= t["o_rel"], f"{what}: {diff}"
    assert diff.lse_max <= t["lse"], f"{what}: {diff}"


def offsets(lens):
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return out


def partial_row(wl, s, b, kappa, r):
    """Workspace row of (sequence s, block b, KV head kappa, query row r) per the ABI layout."""
    g = wl.group
    base = 0
    for t in range(s):
        base += wl.num_blocks(t) * wl.num_kv_heads * wl.q_lens[t] * g
    rows = wl.q_lens[s] * g
    return base + (kappa * wl.num_blocks(s) + b) * rows + r


def assert_fused_matches_merge(wl, plan, out_f, lse_f, out_m, lse_m) -> None:
    """The fused call against partial_attn + merge on the same plan (torch tensors).

    The fused call writes the rows of single-block sequences from its fp32 accumulators;
    the separate merge reads them back from the stored partials. Every LSE and every
    multi-block row is the same bits in both; single-block rows too with fp32 partials.
    With row-scaled fp16 partials a single-block row differs by the element's fp16
    rounding: at most half an fp16 step at 1.0 (2^-12) of the row's largest |O|, plus
    fp32 rounding of the scale (the 1.002 factor)."""
    import torch

    assert torch.equal(lse_f, lse_m), "LSE differs between the fused call and the merge"
    if plan.info()["partial_format"] == 0:
        assert torch.equal(out_f, out_m), "fp32 partials: the fused call and the merge differ"
        return
    single = torch.zeros(wl.total_q, dtype=torch.bool)
    for s, o in enumerate(offsets(wl.q_lens)[:-1]):
        if wl.num_blocks(s) == 1:
            single[o:o + wl.q_lens[s]] = True
    single = single.to(out_f.device)
    assert torch.equal(out_f[~single], out_m[~single]), "multi-block rows differ"
    a, b = out_f[single], out_m[single]
    bound = a.abs().amax(dim=-1, keepdim=True) * (2.0 ** -12 * 1.002)
    assert bool(((a - b).abs() <= bound).all()), "single-block rows beyond the fp16 partial bound"


def scale_of(wl):
    return 1.0 / math.sqrt(wl.head_dim)


def oracle_threads() -> int:
    """Host threads for the oracle: the CPUs this process may use, capped by
    OMP_NUM_THREADS where the environment sets it."""
    import os

    avail = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(avail, int(env))) if env.isdigit() and int(env) > 0 else avail


def compare_whole(wl, q, k, v, out, lse, seqs=None, rows_per_task=2048, threads=None, progress=None) -> Diff:
    """Whole-output parity: the float64 oracle over every (sequence, KV head) of the
    workload (or of ``seqs``), against the device results ``out`` [sum q, Hq, D] and
    ``lse`` [sum q, Hq]. Streams one sequence's K/V at a time to the host; the oracle's
    rows of one KV head are independent, so each (sequence, KV head) is cut into tasks
    of at most ``rows_per_task`` rows that run on a thread pool (BLAS one thread each).
    Returns max|dO|, relative L2 over all compared outputs, and max|dLSE|."""
    import threading
    from concurrent.futures import ThreadPoolExecutor

    import torch

    from oracle import attend_rows

    threads = threads or oracle_threads()
    g, d = wl.group, wl.head_dim
    sc = scale_of(wl)
    qo, ko = offsets(wl.q_lens), offsets(wl.kv_lens)
    seqs = range(wl.batch) if seqs is None else seqs
    o_host = out.detach().cpu().numpy()
    l_host = lse.detach().cpu().numpy()
    acc = {"d2": 0.0, "r2": 0.0, "omax": 0.0, "lmax": 0.0, "n": 0}
    lock = threading.Lock()

    def widen(t):
        return t.to(torch.float32).numpy().astype(np.float64)

    def task(s, kap, r0, r1, qh, kh, vh):
        n, qs = wl.kv_lens[s], wl.q_lens[s]
        Q = widen(qh[:, kap * g:(kap + 1) * g].reshape(qs * g, d)[r0:r1])
        # K and V come widened when the (sequence, KV head) is split into several tasks.
        K, V = (kh, vh) if isinstance(kh, np.ndarray) else (widen(kh[:, kap]), widen(vh[:, kap]))
        pos = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)[r0:r1]
        O, L = attend_rows(Q, pos, K, V, sc, wl.causal)
        go = o_host[qo[s]:qo[s + 1], kap * g:(kap + 1) * g].reshape(qs * g, d)[r0:r1].astype(np.float64)
        gl = l_host[qo[s]:qo[s + 1], kap * g:(kap + 1) * g].reshape(qs * g)[r0:r1].astype(np.float64)
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), f"non-finite output in sequence {s}"
        dd = go - O
        with lock:
            acc["d2"] += float(np.sum(dd * dd))
            acc["r2"] += float(np.sum(O * O))
            acc["omax"] = max(acc["omax"], float(np.max(np.abs(dd))))
            acc["lmax"] = max(acc["lmax"], float(np.max(np.abs(gl - L))))
            acc["n"] += r1 - r0

    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(limits=1, user_api="blas")
    except Exception:
        limiter = None
    try:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            pending = []
            for s in seqs:
                qh = q[qo[s]:qo[s + 1]].detach().cpu()
                kh = k[ko[s]:ko[s + 1]].detach().cpu()
                vh = v[ko[s]:ko[s + 1]].detach().cpu()
                rows = wl.q_lens[s] * g
                for kap in range(wl.num_kv_heads):
                    kk, vv = (widen(kh[:, kap]), widen(vh[:, kap])) if rows > rows_per_task else (kh, vh)
                    for r0 in range(0, rows, rows_per_task):
                        pending.append(ex.submit(task, s, kap, r0, min(rows, r0 + rows_per_task), qh, kk, vv))
                    del kk, vv
                # Bound the host copies in flight.
                while len(pending) > 4 * threads:
                    pending.pop(0).result()
                if progress is not None:
                    progress(s)
            for f in pending:
                f.result()
    finally:
        if limiter is not None:
            limiter.unregister()
    rel = math.sqrt(acc["d2"] / acc["r2"]) if acc["r2"] > 0 else math.sqrt(acc["d2"])
    res = Diff(acc["omax"], rel, acc["lmax"])
    res.d2, res.r2 = acc["d2"], acc["r2"]  # sums of squares, to combine parts of one output
    return res


class GradDiff:
    """Whole-tensor errors of dQ, dK and dV: relative L2 and the largest element error
    relative to the tensor's largest reference magnitude (the backward tolerance's
    two measures), from sums that combine over parts of one tensor."""

    def __init__(self):
        self.acc = {t: {"d2": 0.0, "r2": 0.0, "dmax": 0.0, "rmax": 0.0} for t in ("dq", "dk", "dv")}

    def add(self, name, got, ref):
        a, d = self.acc[name], got - ref
        a["d2"] += float(np.sum(d * d))
        a["r2"] += float(np.sum(ref * ref))
        a["dmax"] = max(a["dmax"], float(np.max(np.abs(d))) if d.size else 0.0)
        a["rmax"] = max(a["rmax"], float(np.max(np.abs(ref))) if ref.size else 0.0)

    def errors(self, name):
        a = self.acc[name]
        return math.sqrt(a["d2"] / max(a["r2"], 1e-300)), a["dmax"] / max(a["rmax"], 1e-30)

    def __str__(self):
        return ", ".join(f"{t}: rel L2 {self.errors(t)[0]:.2e}, max |d| / max |ref| {self.errors(t)[1]:.2e}"
                         for t in ("dq", "dk", "dv"))


def compare_grads_whole(wl, q, k, v, do, out, lse, dq, dk, dv, seqs=None, keys_per_task=16384, threads=None):
    """Whole-tensor backward parity: the float64 oracle's gradients at the device's
    forward outputs (out, lse) for every (sequence, KV head) of the workload (or of
    ``seqs``), against the device gradients dq [sum q, Hq, D] and dk, dv [sum n, Hkv, D]
    (any float dtype). One sequence's tensors are copied to the host at a time; each
    (sequence, KV head) is cut into key ranges that run on a thread pool (BLAS one
    thread each): a range gives its keys' dK and dV and a part of every row's dQ, and
    the parts are summed before dQ is compared. Returns a GradDiff."""
    import threading
    from concurrent.futures import ThreadPoolExecutor

    import torch

    from oracle.backward import grad_rows

    threads = threads or oracle_threads()
    g, d = wl.group, wl.head_dim
    sc = scale_of(wl)
    qo, ko = offsets(wl.q_lens), offsets(wl.kv_lens)
    seqs = range(wl.batch) if seqs is None else seqs
    res = GradDiff()
    lock = threading.Lock()

    def f64(t):  # exact for bf16, fp32 and fp64 tensors
        return t.to(torch.float64).numpy()

    def rows_of(t, kap, qs):
        return t[:, kap * g:(kap + 1) * g].reshape(qs * g, -1) if t.dim() == 3 else t[:, kap * g:(kap + 1) * g].reshape(qs * g)

    def task(s, kap, lo, hi, Q, dO, O, L, pos, kh, vh, gk, gv, dq_part):
        K, V = f64(kh[lo:hi, kap]), f64(vh[lo:hi, kap])
        dqp, dkp, dvp = grad_rows(Q, pos - lo, K, V, dO, O, L, sc, wl.causal)
        gkp, gvp = f64(gk[lo:hi, kap]), f64(gv[lo:hi, kap])
        assert np.all(np.isfinite(gkp)) and np.all(np.isfinite(gvp)), f"non-finite dK/dV in sequence {s}"
        with lock:
            res.add("dk", gkp, dkp)
            res.add("dv", gvp, dvp)
            dq_part += dqp

    try:
        from threadpoolctl import threadpool_limits

        limiter = threadpool_limits(limits=1, user_api="blas")
    except Exception:
        limiter = None
    def finish(s, qs, gq, parts, futs):
        for f in futs:
            f.result()
        for kap, part in enumerate(parts):
            got = f64(rows_of(gq, kap, qs))
            assert np.all(np.isfinite(got)), f"non-finite dQ in sequence {s}"
            res.add("dq", got, part)

    try:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            open_seqs, n_open = [], 0  # sequences whose tasks may still run, oldest first
            for s in seqs:
                n, qs = wl.kv_lens[s], wl.q_lens[s]
                qh, doh = q[qo[s]:qo[s + 1]].detach().cpu(), do[qo[s]:qo[s + 1]].detach().cpu()
                oh, lh = out[qo[s]:qo[s + 1]].detach().cpu(), lse[qo[s]:qo[s + 1]].detach().cpu()
                gq = dq[qo[s]:qo[s + 1]].detach().cpu()
                kh, vh = k[ko[s]:ko[s + 1]].detach().cpu(), v[ko[s]:ko[s + 1]].detach().cpu()
                gk, gv = dk[ko[s]:ko[s + 1]].detach().cpu(), dv[ko[s]:ko[s + 1]].detach().cpu()
                pos = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)
                parts, futs = [], []
                for kap in range(wl.num_kv_heads):
                    Q, dO, O = f64(rows_of(qh, kap, qs)), f64(rows_of(doh, kap, qs)), f64(rows_of(oh, kap, qs))
                    L = f64(rows_of(lh, kap, qs))
                    part = np.zeros((qs * g, d), dtype=np.float64)
                    parts.append(part)
                    for lo in range(0, n, keys_per_task):
                        futs.append(ex.submit(task, s, kap, lo, min(n, lo + keys_per_task), Q, dO, O, L, pos,
                                              kh, vh, gk, gv, part))
                open_seqs.append((s, qs, gq, parts, futs))
                n_open += len(futs)
                # Bound the host copies in flight: finish the oldest sequences first.
                while n_open > 4 * threads and len(open_seqs) > 1:
                    e = open_seqs.pop(0)
                    finish(*e)
                    n_open -= len(e[4])
            for e in open_seqs:
                finish(*e)
    finally:
        if limiter is not None:
            limiter.unregister()
    return res
