"""Exact split-KV attention for AMD MI355X (gfx950).

The computation lives in ``libsplitkv.so`` (C ABI, ``include/splitkv.h``): an LPT
planner on the host and HIP kernels for per-block partial attention, the
log-sum-exp merge, the fused call, and the backward pass. This package is its ctypes
binding.
"""

from .api import (  # noqa: F401
    Plan,
    SplitKVError,
    plan_for,
    splitkv_attn,
    splitkv_attn_backward,
    splitkv_attn_scratch,
    splitkv_merge,
    splitkv_partial_attn,
    splitkv_plan,
    splitkv_plan_upload,
    status_string,
    version,
    workspace,
    workspace_views,
)
from ._lib import SPLITKV_PARTIAL_F16_ROWSCALE, SPLITKV_PARTIAL_F32  # noqa: F401
