"""ctypes declarations of libsplitkv's C ABI (include/splitkv.h).

Loading the library touches no GPU. There is no fallback: if the library has not
been built, ``load()`` raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsplitkv.so")

SPLITKV_OK = 0
SPLITKV_ERR_INVALID_ARG = -1
SPLITKV_ERR_UNSUPPORTED = -2
SPLITKV_ERR_WORKSPACE = -3
SPLITKV_ERR_HIP = -4
SPLITKV_ERR_ALLOC = -5

SPLITKV_F32 = 0
SPLITKV_BF16 = 1

SPLITKV_UNIT_SEQ_BLOCK_KVHEAD = 0
SPLITKV_UNIT_SEQ_BLOCK = 1

SPLITKV_SCRATCH_BYTES = 256 << 20

SPLITKV_SCHED_AUTO = 0
SPLITKV_SCHED_QUEUE = 1
SPLITKV_SCHED_STATIC = 2

SPLITKV_PARTIAL_F32 = 0
SPLITKV_PARTIAL_F16_ROWSCALE = 1

# Every function include/splitkv.h declares.
EXPORTED = (
    "splitkv_version",
    "splitkv_plan",
    "splitkv_plan_info_get",
    "splitkv_plan_export",
    "splitkv_plan_upload",
    "splitkv_plan_destroy",
    "splitkv_partial_attn",
    "splitkv_merge",
    "splitkv_attn",
    "splitkv_attn_scratch",
    "splitkv_attn_backward",
    "splitkv_status_string",
    "splitkv_last_error",
)


class Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("kv_lens", ctypes.POINTER(ctypes.c_int64)),
        ("q_lens", ctypes.POINTER(ctypes.c_int32)),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
        ("num_workers", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("granularity", ctypes.c_int32),
        ("cost_ridge_rows", ctypes.c_int32),
        ("xcd_speed", ctypes.POINTER(ctypes.c_int32)),
        ("partial_format", ctypes.c_int32),
    ]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("num_units", ctypes.c_int64),
        ("total_cost", ctypes.c_int64),
        ("makespan", ctypes.c_int64),
        ("lower_bound", ctypes.c_int64),
        ("imbalance", ctypes.c_double),
        ("total_q", ctypes.c_int64),
        ("total_kv", ctypes.c_int64),
        ("partial_rows", ctypes.c_int64),
        ("plan_bytes", ctypes.c_size_t),
        ("workspace_bytes", ctypes.c_size_t),
        ("ws_lse_offset", ctypes.c_size_t),
        ("num_jobs", ctypes.c_int64),
        ("exec_imbalance_static", ctypes.c_double),
        ("exec_imbalance_static_est", ctypes.c_double),
        ("exec_imbalance_queue_est", ctypes.c_double),
        ("auto_schedule", ctypes.c_int32),
        ("num_mma_jobs", ctypes.c_int64),
        ("mma_partial_passes", ctypes.c_int32),
        ("partial_format", ctypes.c_int32),
    ]


class Inputs(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("q_stride_tok", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("k_stride_tok", ctypes.c_int64),
        ("k_stride_head", ctypes.c_int64),
        ("v_stride_tok", ctypes.c_int64),
        ("v_stride_head", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("schedule", ctypes.c_int32),
        ("worker_clock", ctypes.c_void_p),
    ]


class Grads(ctypes.Structure):
    _fields_ = [
        ("d_out", ctypes.c_void_p),
        ("do_stride_tok", ctypes.c_int64),
        ("do_stride_head", ctypes.c_int64),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("dkv_dtype", ctypes.c_int32),
    ]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libsplitkv.so (built in-tree by split_kv_exact_amd.build)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m split_kv_exact_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    i32p, i64p = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)
    sig = {
        "splitkv_version": (ctypes.c_int, []),
        "splitkv_plan": (ctypes.c_int, [ctypes.POINTER(Problem), ctypes.POINTER(P)]),
        "splitkv_plan_info_get": (ctypes.c_int, [P, ctypes.POINTER(PlanInfo)]),
        "splitkv_plan_export": (ctypes.c_int, [P, i32p, i32p, i32p, i32p, i64p, i32p, i32p, i32p, i64p]),
        "splitkv_plan_upload": (ctypes.c_int, [P, P, ctypes.c_size_t, P]),
        "splitkv_plan_destroy": (None, [P]),
        "splitkv_partial_attn": (ctypes.c_int, [P, P, ctypes.POINTER(Inputs), P, ctypes.c_size_t, P]),
        "splitkv_merge": (ctypes.c_int, [P, P, P, ctypes.c_size_t, P, P, P]),
        "splitkv_attn": (ctypes.c_int, [P, P, ctypes.POINTER(Inputs), P, ctypes.c_size_t, P, P, P]),
        "splitkv_attn_scratch": (ctypes.c_int, [P, P, ctypes.POINTER(Inputs), P, P, P]),
        "splitkv_attn_backward": (ctypes.c_int, [P, P, ctypes.POINTER(Inputs), ctypes.POINTER(Grads), P,
                                                 ctypes.c_size_t, P]),
        "splitkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "splitkv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib
