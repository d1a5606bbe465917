"""Thin Python binding of libsplitkv: the same calls as include/splitkv.h.

Argument marshalling only. PyTorch provides device memory and the current stream;
every step of the computation runs in the library's HIP kernels. Errors from the
library raise ``SplitKVError`` with the library's status and detail text.
"""

from __future__ import annotations

import ctypes
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

from . import _lib as L


class SplitKVError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {detail or 'error'} (status {status})")


def _check(lib, status: int, where: str) -> None:
    if status != L.SPLITKV_OK:
        raise SplitKVError(status, where, lib.splitkv_last_error().decode())


class Plan:
    """An LPT plan (library-owned host object) and the problem it was made for."""

    def __init__(self, handle, problem: dict, lib):
        self._h = handle
        self._lib = lib
        self.problem = problem

    @property
    def handle(self):
        return self._h

    def info(self) -> Dict[str, object]:
        inf = L.PlanInfo()
        _check(self._lib, self._lib.splitkv_plan_info_get(self._h, ctypes.byref(inf)), "splitkv_plan_info_get")
        return {name: getattr(inf, name) for name, _ in L.PlanInfo._fields_}

    def export(self) -> Dict[str, np.ndarray]:
        inf = self.info()
        n, m = int(inf["num_units"]), int(self.problem["num_workers"])
        out = {
            "unit_seq": np.zeros(n, np.int32),
            "unit_block": np.zeros(n, np.int32),
            "unit_kv_head": np.zeros(n, np.int32),
            "unit_len": np.zeros(n, np.int32),
            "unit_cost": np.zeros(n, np.int64),
            "worker_of": np.zeros(n, np.int32),
            "worker_ptr": np.zeros(m + 1, np.int32),
            "worker_units": np.zeros(n, np.int32),
            "load": np.zeros(m, np.int64),
        }
        ptrs = [out[k].ctypes.data_as(ctypes.POINTER(ctypes.c_int64 if out[k].dtype == np.int64 else ctypes.c_int32))
                for k in ("unit_seq", "unit_block", "unit_kv_head", "unit_len", "unit_cost", "worker_of",
                          "worker_ptr", "worker_units", "load")]
        _check(self._lib, self._lib.splitkv_plan_export(self._h, *ptrs), "splitkv_plan_export")
        return out

    def close(self) -> None:
        if self._h:
            self._lib.splitkv_plan_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def splitkv_plan(
    kv_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_len: int,
    num_workers: int,
    causal: bool = True,
    granularity: int = L.SPLITKV_UNIT_SEQ_BLOCK_KVHEAD,
    cost_ridge_rows: int = 0,
    xcd_speed: Sequence[int] | None = None,
    partial_format: int = L.SPLITKV_PARTIAL_F32,
) -> Plan:
    """Build the LPT plan on the host (``splitkv_plan``). ``cost_ridge_rows`` selects the
    unit cost: 0 is q * len * heads, R > 0 is len * max(q * g, R) per KV head.
    ``xcd_speed`` (8 relative speeds, or None) places the most loaded workers on the
    workgroups of the fastest XCDs. ``partial_format``: how the per-block partials are
    stored (``SPLITKV_PARTIAL_F32``, or ``SPLITKV_PARTIAL_F16_ROWSCALE`` for bf16 inputs,
    half the bytes)."""
    lib = L.load()
    kv = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int64))
    ql = np.ascontiguousarray(np.asarray(q_lens, dtype=np.int32))
    prob = L.Problem(
        batch=len(kv),
        kv_lens=kv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
        q_lens=ql.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        block_len=block_len,
        num_workers=num_workers,
        causal=int(bool(causal)),
        granularity=granularity,
        cost_ridge_rows=cost_ridge_rows,
        partial_format=partial_format,
    )
    speeds = None
    if xcd_speed is not None:
        speeds = np.ascontiguousarray(np.asarray(xcd_speed, dtype=np.int32))
        if speeds.shape != (8,):
            raise ValueError("xcd_speed must hold 8 values")
        prob.xcd_speed = speeds.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    h = ctypes.c_void_p()
    _check(lib, lib.splitkv_plan(ctypes.byref(prob), ctypes.byref(h)), "splitkv_plan")
    problem = dict(kv_lens=kv.tolist(), q_lens=ql.tolist(), num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
                   head_dim=head_dim, block_len=block_len, num_workers=num_workers, causal=bool(causal),
                   granularity=granularity, cost_ridge_rows=cost_ridge_rows,
                   xcd_speed=None if speeds is None else speeds.tolist(), partial_format=partial_format)
    return Plan(h, problem, lib)


def plan_for(wl, cost_ridge_rows: int = 0, xcd_speed: Sequence[int] | None = None,
             partial_format: int | None = None) -> Plan:
    """Plan for a ``workloads.Workload``; its partials are row-scaled fp16 for bf16
    inputs and fp32 for fp32 inputs unless ``partial_format`` says otherwise."""
    if partial_format is None:
        partial_format = L.SPLITKV_PARTIAL_F16_ROWSCALE if wl.dtype == "bfloat16" else L.SPLITKV_PARTIAL_F32
    return splitkv_plan(wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.head_dim, wl.block_len,
                        wl.num_workers, wl.causal, wl.granularity, cost_ridge_rows, xcd_speed, partial_format)


# --------------------------------------------------------------------------- device side

def _torch():
    import torch

    return torch


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def splitkv_plan_upload(plan: Plan, device=None, stream=None):
    """Copy the plan's device image into a new uint8 device tensor (``splitkv_plan_upload``)."""
    torch = _torch()
    inf = plan.info()
    buf = torch.empty(int(inf["plan_bytes"]), dtype=torch.uint8, device=device or "cuda")
    _check(plan._lib, plan._lib.splitkv_plan_upload(plan.handle, ctypes.c_void_p(buf.data_ptr()), buf.numel(),
                                                    _stream(stream)), "splitkv_plan_upload")
    return buf


def workspace(plan: Plan, device=None):
    torch = _torch()
    nbytes = int(plan.info()["workspace_bytes"])
    return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=device or "cuda")


def workspace_views(plan: Plan, ws) -> Tuple[object, object]:
    """(partial outputs [partial_rows, D], partial LSEs [partial_rows]) of a workspace, as
    fp32: views for fp32 partials; for row-scaled fp16 partials, new tensors holding each
    element times its row's scale."""
    torch = _torch()
    inf = plan.info()
    rows, d = int(inf["partial_rows"]), int(plan.problem["head_dim"])
    off = int(inf["ws_lse_offset"]) // 4
    if int(inf["partial_format"]) == L.SPLITKV_PARTIAL_F32:
        return ws[: rows * d].view(rows, d), ws[off: off + rows]
    h = ws[: (rows * d + 1) // 2].view(torch.float16)[: rows * d].view(rows, d)
    pairs = ws[off: off + 2 * rows].view(rows, 2)
    return h.float() * pairs[:, 1:2], pairs[:, 0].clone()


_SCHEDULES = {"auto": L.SPLITKV_SCHED_AUTO, "queue": L.SPLITKV_SCHED_QUEUE, "static": L.SPLITKV_SCHED_STATIC}


def _inputs(q, k, v, scale: float, schedule: str = "auto", clock=None) -> L.Inputs:
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be [tokens, heads, head_dim] with contiguous head_dim")
    if not (q.dtype == k.dtype == v.dtype):
        raise ValueError("q, k and v must share a dtype")
    if q.dtype == torch.bfloat16:
        dt = L.SPLITKV_BF16
    elif q.dtype == torch.float32:
        dt = L.SPLITKV_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    return L.Inputs(
        q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(),
        q_stride_tok=q.stride(0), q_stride_head=q.stride(1),
        k_stride_tok=k.stride(0), k_stride_head=k.stride(1),
        v_stride_tok=v.stride(0), v_stride_head=v.stride(1),
        dtype=dt, scale=float(scale),
        schedule=_SCHEDULES[schedule] if schedule in _SCHEDULES else int(schedule),
        worker_clock=None if clock is None else clock.data_ptr(),
    )


def _check_shapes(plan: Plan, q, k, v) -> None:
    p = plan.problem
    tq, tk = sum(p["q_lens"]), sum(p["kv_lens"])
    if tuple(q.shape) != (tq, p["num_q_heads"], p["head_dim"]):
        raise ValueError(f"q has shape {tuple(q.shape)}, plan expects {(tq, p['num_q_heads'], p['head_dim'])}")
    for name, t in (("k", k), ("v", v)):
        if tuple(t.shape) != (tk, p["num_kv_heads"], p["head_dim"]):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, plan expects {(tk, p['num_kv_heads'], p['head_dim'])}")


def splitkv_partial_attn(plan: Plan, dev_plan, q, k, v, ws=None, scale: float = 0.0, stream=None,
                         schedule: str = "auto", clock=None):
    """Per-block partial outputs and LSEs into the workspace (``splitkv_partial_attn``).

    ``schedule`` is "auto", "queue" (the cheapest jobs form a tail shared at run
    time) or "static" (each workgroup runs its plan worker's units); ``clock`` is
    None or an int64 device tensor of
    2 * num_workers entries that receives each workgroup's start and end clock."""
    _check_shapes(plan, q, k, v)
    if ws is None:
        ws = workspace(plan, q.device)
    inp = _inputs(q, k, v, scale, schedule, clock)
    _check(plan._lib, plan._lib.splitkv_partial_attn(plan.handle, ctypes.c_void_p(dev_plan.data_ptr()),
                                                     ctypes.byref(inp), ctypes.c_void_p(ws.data_ptr()),
                                                     ws.numel() * ws.element_size(), _stream(stream)),
           "splitkv_partial_attn")
    return ws


def _outputs(plan: Plan, device, out, lse):
    torch = _torch()
    p = plan.problem
    tq = sum(p["q_lens"])
    if out is None:
        out = torch.empty((tq, p["num_q_heads"], p["head_dim"]), dtype=torch.float32, device=device)
    if lse is None:
        lse = torch.empty((tq, p["num_q_heads"]), dtype=torch.float32, device=device)
    if out.dtype != torch.float32 or lse.dtype != torch.float32 or not out.is_contiguous() or not lse.is_contiguous():
        raise ValueError("out and lse must be contiguous float32 tensors")
    if tuple(out.shape) != (tq, p["num_q_heads"], p["head_dim"]) or tuple(lse.shape) != (tq, p["num_q_heads"]):
        raise ValueError("out/lse shapes do not match the plan")
    return out, lse


def splitkv_merge(plan: Plan, dev_plan, ws, out=None, lse=None, stream=None):
    """Log-sum-exp merge of the workspace partials (``splitkv_merge``)."""
    out, lse = _outputs(plan, ws.device, out, lse)
    _check(plan._lib, plan._lib.splitkv_merge(plan.handle, ctypes.c_void_p(dev_plan.data_ptr()),
                                              ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                              ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                              _stream(stream)),
           "splitkv_merge")
    return out, lse


def splitkv_attn(plan: Plan, dev_plan, q, k, v, ws=None, out=None, lse=None, scale: float = 0.0, stream=None,
                 schedule: str = "auto", clock=None):
    """Fused partial attention + merge (``splitkv_attn``); ``schedule`` and ``clock`` as
    for :func:`splitkv_partial_attn`."""
    _check_shapes(plan, q, k, v)
    if ws is None:
        ws = workspace(plan, q.device)
    out, lse = _outputs(plan, q.device, out, lse)
    inp = _inputs(q, k, v, scale, schedule, clock)
    _check(plan._lib, plan._lib.splitkv_attn(plan.handle, ctypes.c_void_p(dev_plan.data_ptr()), ctypes.byref(inp),
                                             ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size(),
                                             ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                                             _stream(stream)),
           "splitkv_attn")
    return out, lse


def splitkv_attn_scratch(plan: Plan, dev_plan, q, k, v, out=None, lse=None, scale: float = 0.0, stream=None,
                         schedule: str = "auto", clock=None):
    """Fused partial attention + merge with the library's own device workspace
    (``splitkv_attn_scratch``): no workspace argument, nothing allocated by the call.
    Calls that overlap in time on one GPU share that workspace and race."""
    _check_shapes(plan, q, k, v)
    out, lse = _outputs(plan, q.device, out, lse)
    inp = _inputs(q, k, v, scale, schedule, clock)
    _check(plan._lib, plan._lib.splitkv_attn_scratch(plan.handle, ctypes.c_void_p(dev_plan.data_ptr()),
                                                     ctypes.byref(inp), ctypes.c_void_p(out.data_ptr()),
                                                     ctypes.c_void_p(lse.data_ptr()), _stream(stream)),
           "splitkv_attn_scratch")
    return out, lse


def splitkv_attn_backward(plan: Plan, dev_plan, q, k, v, do, out, lse, ws=None, dq=None, dk=None, dv=None,
                          scale: float = 0.0, stream=None, dkv_dtype=None):
    """Gradients dQ, dK, dV of sum(do * out) at the forward's ``out`` and ``lse``
    (``splitkv_attn_backward``; bf16 inputs). dQ is float32; dK and dV are float32 or
    bfloat16 (``dkv_dtype``, else the dtype of a given ``dk``, else float32)."""
    torch = _torch()
    _check_shapes(plan, q, k, v)
    if do.shape != q.shape or do.dtype != q.dtype or do.stride(2) != 1:
        raise ValueError("do must match q in shape and dtype, with contiguous head_dim")
    for name, t in (("out", out), ("lse", lse)):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 tensor")
    if ws is None:
        ws = workspace(plan, q.device)
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dkv_dtype is None:
        dkv_dtype = dk.dtype if dk is not None else torch.float32
    if dkv_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("dkv_dtype must be torch.float32 or torch.bfloat16")
    if dk is None:
        dk = torch.empty(k.shape, dtype=dkv_dtype, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=dkv_dtype, device=q.device)
    for name, t, ref, dt in (("dq", dq, q, torch.float32), ("dk", dk, k, dkv_dtype), ("dv", dv, v, dkv_dtype)):
        if t.shape != ref.shape or t.dtype != dt or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {dt} tensor shaped like {name[1]}")
    inp = _inputs(q, k, v, scale)
    gr = L.Grads(d_out=do.data_ptr(), do_stride_tok=do.stride(0), do_stride_head=do.stride(1), out=out.data_ptr(),
                 lse=lse.data_ptr(), dq=dq.data_ptr(), dk=dk.data_ptr(), dv=dv.data_ptr(),
                 dkv_dtype=L.SPLITKV_BF16 if dkv_dtype == torch.bfloat16 else L.SPLITKV_F32)
    _check(plan._lib, plan._lib.splitkv_attn_backward(plan.handle, ctypes.c_void_p(dev_plan.data_ptr()),
                                                      ctypes.byref(inp), ctypes.byref(gr),
                                                      ctypes.c_void_p(ws.data_ptr()),
                                                      ws.numel() * ws.element_size(), _stream(stream)),
           "splitkv_attn_backward")
    return dq, dk, dv


def status_string(status: int) -> str:
    return L.load().splitkv_status_string(status).decode()


def version() -> Tuple[int, int]:
    v = L.load().splitkv_version()
    return v >> 16, v & 0xFFFF
