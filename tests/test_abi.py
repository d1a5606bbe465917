"""C-ABI checks that need no GPU: exports, status strings and argument errors.

Every argument error is reported before the library makes a HIP call, so these run
on a machine without a GPU. Device pointers passed here are never dereferenced.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from split_kv_exact_amd import _lib as L
from split_kv_exact_amd import SplitKVError, splitkv_plan

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "splitkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(splitkv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    decl = declared_functions()
    assert set(decl) == set(L.EXPORTED), decl
    for name in decl:
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    v = lib.splitkv_version()
    assert v >> 16 == 0 and (v & 0xFFFF) >= 1
    assert lib.splitkv_status_string(0) == b"ok"
    for code in (-1, -2, -3, -4, -5):
        s = lib.splitkv_status_string(code)
        assert s and s != b"unknown status"
    assert lib.splitkv_status_string(-99) == b"unknown status"


def _problem(kv, q, hq=4, hkv=2, d=128, b=64, m=8, causal=1, gran=0, ridge=0, speeds=None):
    kv = np.asarray(kv, np.int64)
    q = np.asarray(q, np.int32)
    p = L.Problem(batch=len(kv), kv_lens=kv.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                  q_lens=q.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), num_q_heads=hq, num_kv_heads=hkv,
                  head_dim=d, block_len=b, num_workers=m, causal=causal, granularity=gran, cost_ridge_rows=ridge)
    keep = (kv, q)
    if speeds is not None:
        sp = np.asarray(speeds, np.int32)
        p.xcd_speed = sp.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        keep = (kv, q, sp)
    return p, keep


@pytest.mark.parametrize("kw", [
    dict(kv=[10], q=[0]),            # q_len < 1
    dict(kv=[3], q=[4]),             # kv_len < q_len
    dict(kv=[10], q=[2], hq=6, hkv=4),  # Hq % Hkv != 0
    dict(kv=[10], q=[2], b=0),       # block_len < 1
    dict(kv=[10], q=[2], m=0),       # num_workers < 1
    dict(kv=[10], q=[2], causal=2),
    dict(kv=[10], q=[2], gran=7),
    dict(kv=[10], q=[2], speeds=[1, 1, 1, 0, 1, 1, 1, 1]),  # an XCD speed below 1
    dict(kv=[10], q=[2], ridge=-1),  # negative ridge
    dict(kv=[10], q=[2], ridge=(1 << 30) + 1),
    dict(kv=[1 << 40], q=[1 << 20], hq=1024, hkv=1, b=1 << 30),  # total cost beyond 2^62
    dict(kv=[10], q=[2], hq=0),
    # Block, unit and job indices are int32: 2^40 one-token blocks, or 2^31 units over
    # two KV heads, are rejected before anything is allocated.
    dict(kv=[1 << 40], q=[1], hq=1, hkv=1, b=1),
    dict(kv=[1 << 30], q=[1], hq=2, hkv=2, b=1),
    dict(kv=[1 << 30], q=[1], hq=2, hkv=2, b=1, gran=1, m=1 << 20),
])
def test_invalid_problems_are_rejected(lib, kw):
    p, keep = _problem(**kw)
    h = ctypes.c_void_p(1234)
    st = lib.splitkv_plan(ctypes.byref(p), ctypes.byref(h))
    assert st == L.SPLITKV_ERR_INVALID_ARG
    assert h.value is None
    assert lib.splitkv_last_error()


def test_null_arguments(lib):
    h = ctypes.c_void_p()
    assert lib.splitkv_plan(None, ctypes.byref(h)) == L.SPLITKV_ERR_INVALID_ARG
    p, keep = _problem([10], [2])
    assert lib.splitkv_plan(ctypes.byref(p), None) == L.SPLITKV_ERR_INVALID_ARG
    p.batch = 0
    assert lib.splitkv_plan(ctypes.byref(p), ctypes.byref(h)) == L.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_plan_info_get(None, ctypes.byref(L.PlanInfo())) == L.SPLITKV_ERR_INVALID_ARG
    lib.splitkv_plan_destroy(None)  # ignored


def test_python_binding_raises():
    with pytest.raises(SplitKVError) as e:
        splitkv_plan([5], [9], 4, 2, 128, 16, 4)
    assert e.value.status == L.SPLITKV_ERR_INVALID_ARG
    assert "kv_len" in str(e.value)


FAKE = 1 << 20  # aligned, never dereferenced: every call below fails validation first


def _plan_handle(lib, d=128):
    p, keep = _problem([100, 40], [3, 1], d=d)
    h = ctypes.c_void_p()
    assert lib.splitkv_plan(ctypes.byref(p), ctypes.byref(h)) == 0
    inf = L.PlanInfo()
    assert lib.splitkv_plan_info_get(h, ctypes.byref(inf)) == 0
    return h, inf


def _inputs(dtype=L.SPLITKV_BF16, ptr=FAKE, strides=(256, 128, 256, 128, 256, 128), scale=0.0,
            schedule=L.SPLITKV_SCHED_AUTO, clock=None):
    return L.Inputs(q=ptr, k=ptr, v=ptr, q_stride_tok=strides[0], q_stride_head=strides[1],
                    k_stride_tok=strides[2], k_stride_head=strides[3], v_stride_tok=strides[4],
                    v_stride_head=strides[5], dtype=dtype, scale=scale, schedule=schedule, worker_clock=clock)


def test_partial_attn_argument_errors(lib):
    h, inf = _plan_handle(lib)
    ws, nbytes = ctypes.c_void_p(FAKE), inf.workspace_bytes
    dp = ctypes.c_void_p(FAKE)
    good = _inputs()
    f = lib.splitkv_partial_attn
    assert f(None, dp, ctypes.byref(good), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, None, ctypes.byref(good), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, ctypes.c_void_p(FAKE + 4), ctypes.byref(good), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, None, ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(dtype=5)), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(ptr=0)), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(ptr=FAKE + 2)), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(strides=(256, 100, 256, 128, 256, 128))), ws, nbytes,
             None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(scale=-1.0)), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(scale=float("nan"))), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(good), None, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(schedule=3)), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert b"schedule" in lib.splitkv_last_error()
    assert f(h, dp, ctypes.byref(_inputs(clock=FAKE + 4)), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert b"worker_clock" in lib.splitkv_last_error()
    big = 1 << 25  # bf16 kernels address a stage with 32-bit offsets: strides above 2^24 are refused
    assert f(h, dp, ctypes.byref(_inputs(strides=(big, 128, 256, 128, 256, 128))), ws, nbytes,
             None) == L.SPLITKV_ERR_UNSUPPORTED
    assert f(h, dp, ctypes.byref(good), ws, nbytes - 1, None) == L.SPLITKV_ERR_WORKSPACE
    assert b"workspace needs" in lib.splitkv_last_error()
    lib.splitkv_plan_destroy(h)


def test_unsupported_head_dim(lib):
    h, inf = _plan_handle(lib, d=96)
    st = lib.splitkv_partial_attn(h, ctypes.c_void_p(FAKE), ctypes.byref(_inputs()), ctypes.c_void_p(FAKE),
                                  inf.workspace_bytes, None)
    assert st == L.SPLITKV_ERR_UNSUPPORTED
    lib.splitkv_plan_destroy(h)


def test_merge_and_attn_argument_errors(lib):
    h, inf = _plan_handle(lib)
    dp, ws, nbytes = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), inf.workspace_bytes
    out, lse = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE)
    assert lib.splitkv_merge(h, dp, ws, nbytes, None, lse, None) == L.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_merge(h, dp, ws, nbytes, ctypes.c_void_p(FAKE + 8), lse, None) == L.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_merge(h, dp, ws, 16, out, lse, None) == L.SPLITKV_ERR_WORKSPACE
    good = _inputs()
    assert lib.splitkv_attn(h, dp, ctypes.byref(good), ws, nbytes, out, None, None) == L.SPLITKV_ERR_INVALID_ARG
    assert lib.splitkv_attn(h, dp, ctypes.byref(good), ws, 0, out, lse, None) == L.SPLITKV_ERR_WORKSPACE
    assert lib.splitkv_plan_upload(h, dp, inf.plan_bytes - 1, None) == L.SPLITKV_ERR_WORKSPACE
    assert lib.splitkv_plan_upload(h, None, inf.plan_bytes, None) == L.SPLITKV_ERR_INVALID_ARG
    lib.splitkv_plan_destroy(h)


def test_backward_argument_errors(lib):
    h, inf = _plan_handle(lib)
    dp, ws, nbytes = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), inf.workspace_bytes
    f = lib.splitkv_attn_backward

    def grads(**kw):
        g = dict(d_out=FAKE, do_stride_tok=256, do_stride_head=128, out=FAKE, lse=FAKE, dq=FAKE, dk=FAKE, dv=FAKE)
        g.update(kw)
        return L.Grads(**g)

    good = _inputs()
    assert f(h, dp, ctypes.byref(good), None, ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(_inputs(dtype=L.SPLITKV_F32)), ctypes.byref(grads()), ws, nbytes,
             None) == L.SPLITKV_ERR_UNSUPPORTED
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads(d_out=0)), ws, nbytes, None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads(dk=FAKE + 4)), ws, nbytes,
             None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads(lse=FAKE + 2)), ws, nbytes,
             None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads(do_stride_head=100)), ws, nbytes,
             None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads(do_stride_tok=1 << 25)), ws, nbytes,
             None) == L.SPLITKV_ERR_UNSUPPORTED
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads(dkv_dtype=2)), ws, nbytes,
             None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads(dkv_dtype=-1)), ws, nbytes,
             None) == L.SPLITKV_ERR_INVALID_ARG
    assert f(h, dp, ctypes.byref(good), ctypes.byref(grads()), ws, 16, None) == L.SPLITKV_ERR_WORKSPACE
    lib.splitkv_plan_destroy(h)


def test_plan_info_sizes():
    pl = splitkv_plan([100, 40], [3, 1], 4, 2, 128, 64, 8)
    inf = pl.info()
    g = 2
    rows = 2 * (2 * 3 * g) + 1 * (2 * 1 * g)  # nb * Hkv * q * g per sequence
    assert inf["partial_rows"] == rows
    assert inf["ws_lse_offset"] == rows * 128 * 4
    assert inf["workspace_bytes"] >= rows * 129 * 4
    assert inf["total_q"] == 4 and inf["total_kv"] == 140
    assert inf["plan_bytes"] > 0 and inf["plan_bytes"] % 16 == 0


def test_workspace_holds_the_backward_row_values():
    """The backward pass keeps two floats per (query token, query head) in the LSE area
    (D and the LSE in base 2). With one block per sequence the partial rows are exactly
    sum q * Hq, half of that: the workspace grows to hold both."""
    pl = splitkv_plan([50, 64], [7, 3], 8, 2, 128, 64, 8)  # one block each
    inf = pl.info()
    qh = 10 * 8
    assert inf["partial_rows"] == qh
    assert inf["workspace_bytes"] >= inf["ws_lse_offset"] + 2 * qh * 4
    many = splitkv_plan([640, 320], [7, 3], 8, 2, 128, 64, 8).info()  # 10 and 5 blocks
    assert many["workspace_bytes"] == many["ws_lse_offset"] + 4 * many["partial_rows"]


def test_partial_formats():
    """Row-scaled fp16 partials keep an (LSE, scale) pair per row: the LSE area doubles,
    the element area keeps its fp32 size (the backward pass stores fp32 parts there)."""
    f32 = splitkv_plan([640, 320], [7, 3], 8, 2, 128, 64, 8).info()
    h16 = splitkv_plan([640, 320], [7, 3], 8, 2, 128, 64, 8,
                       partial_format=L.SPLITKV_PARTIAL_F16_ROWSCALE).info()
    assert f32["partial_format"] == L.SPLITKV_PARTIAL_F32
    assert h16["partial_format"] == L.SPLITKV_PARTIAL_F16_ROWSCALE
    assert h16["partial_rows"] == f32["partial_rows"] and h16["ws_lse_offset"] == f32["ws_lse_offset"]
    assert h16["workspace_bytes"] == h16["ws_lse_offset"] + 8 * h16["partial_rows"]
    with pytest.raises(SplitKVError) as e:
        splitkv_plan([10], [2], 4, 2, 128, 64, 8, partial_format=2)
    assert e.value.status == L.SPLITKV_ERR_INVALID_ARG and "partial_format" in str(e.value)


def test_fp32_inputs_need_fp32_partials(lib):
    p, keep = _problem([100, 40], [3, 1])
    p.partial_format = L.SPLITKV_PARTIAL_F16_ROWSCALE
    h = ctypes.c_void_p()
    assert lib.splitkv_plan(ctypes.byref(p), ctypes.byref(h)) == 0
    inf = L.PlanInfo()
    assert lib.splitkv_plan_info_get(h, ctypes.byref(inf)) == 0
    ws, dp = ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE)
    st = lib.splitkv_partial_attn(h, dp, ctypes.byref(_inputs(dtype=L.SPLITKV_F32)), ws, inf.workspace_bytes, None)
    assert st == L.SPLITKV_ERR_UNSUPPORTED and b"partial_format" in lib.splitkv_last_error()
    lib.splitkv_plan_destroy(h)


@pytest.mark.parametrize("q, g, jobs, partial", [
    ([3, 1], 2, False, 0),          # every job below 8 row tiles: no matrix-path launch
    ([64, 125, 20], 4, True, 0),    # 256 and 500 rows: passes of 16 tiles only
    ([300], 4, True, 1),            # 1200 rows: five passes of 15 tiles
    ([64, 32], 4, True, 1),         # 128 rows: a pass of 8 tiles
])
def test_matrix_path_passes(q, g, jobs, partial):
    """Jobs of >= 8 row tiles go to the matrix-path launch; its kernel variant with
    per-wave tile skipping runs only when some pass has fewer than 16 tiles."""
    kv = [max(4 * x, 64) for x in q]
    pl = splitkv_plan(kv, q, 8 * g, 8, 128, 512, 16)
    inf = pl.info()
    assert (inf["num_mma_jobs"] > 0) == jobs
    assert inf["mma_partial_passes"] == partial
