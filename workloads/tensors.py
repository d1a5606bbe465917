"""Seeded Q/K/V tensors for a workload.

Layout (shared by every consumer): Q is ``[sum_s q_s, Hq, D]`` and K, V are
``[sum_s n_s, Hkv, D]``, packed by sequence in batch order. Values are standard
normal fp32 draws from a seeded ``torch.Generator`` on the target device, in the
order q, then k (with its boost mask, chunk by chunk), then v, and are then rounded
to the workload dtype (bf16 rounding is round-to-nearest-even).

Random streams differ between the CPU and GPU generators, so a parity check draws
on the device once and hands the oracle a host copy.
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import Workload

_DTYPES = {"float32": torch.float32, "bfloat16": torch.bfloat16}

# Tokens drawn per chunk for K and V, bounding the fp32 temporary (~0.5 GiB at 8x128).
_CHUNK_TOKENS = 1 << 17


def torch_dtype(wl: Workload) -> torch.dtype:
    return _DTYPES[wl.dtype]


def make_qkv(wl: Workload, device="cpu", seed: int | None = None):
    """Return (q, k, v) torch tensors of ``wl.dtype`` on ``device``."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(int(wl.seed if seed is None else seed))
    dt = torch_dtype(wl)
    hq, hkv, d = wl.num_q_heads, wl.num_kv_heads, wl.head_dim
    q = torch.randn((wl.total_q, hq, d), generator=gen, device=dev, dtype=torch.float32).to(dt)
    k = torch.empty((wl.total_kv, hkv, d), device=dev, dtype=dt)
    v = torch.empty((wl.total_kv, hkv, d), device=dev, dtype=dt)
    n = wl.total_kv
    for t0 in range(0, n, _CHUNK_TOKENS):
        t1 = min(n, t0 + _CHUNK_TOKENS)
        kc = torch.randn((t1 - t0, hkv, d), generator=gen, device=dev, dtype=torch.float32)
        if wl.boost_frac > 0.0:
            mask = torch.rand((t1 - t0, hkv), generator=gen, device=dev) < wl.boost_frac
            kc = torch.where(mask[..., None], kc * wl.boost, kc)
        k[t0:t1] = kc.to(dt)
        del kc
    for t0 in range(0, n, _CHUNK_TOKENS):
        t1 = min(n, t0 + _CHUNK_TOKENS)
        v[t0:t1] = torch.randn((t1 - t0, hkv, d), generator=gen, device=dev, dtype=torch.float32).to(dt)
    return q, k, v


def widen_to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a bf16/fp32 tensor to a host float64 numpy array."""
    return t.detach().to("cpu").to(torch.float32).numpy().astype(np.float64)


def seq_offsets(lens) -> np.ndarray:
    """Exclusive prefix sums: token offset of each sequence in the packed layout."""
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return out
