"""Seeded synthetic workloads for exact split-KV attention.

This module is shared by the tests, the benchmark and the oracle-side checks. It
holds only problem shapes and seeded random draws: no attention, merge or
planning arithmetic lives here, so the oracle and the HIP path stay independent.
"""

from .configs import (  # noqa: F401
    Workload,
    WORKLOADS,
    get_workload,
    small_fp32,
    batch8_bf16,
    long_context_bf16,
    lognormal_mix_bf16,
    mixed_decode_prefill_bf16,
    decode_only_bf16,
)
from .tensors import make_qkv, widen_to_f64  # noqa: F401
