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


def scale_of(wl):
    return 1.0 / math.sqrt(wl.head_dim)
