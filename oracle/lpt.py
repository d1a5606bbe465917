"""Pure-Python longest-processing-time-first (LPT) plan for split-KV units.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Split-KV page ("Timeline") places context KV blocks on workers with a cost-aware
LPT strategy and reports a load-imbalance rate below 1%. It gives neither the cost
nor the tie-breaks nor the definition of the rate; the readings here are:

* Unit: (sequence s, block b, KV head kappa), enumerated in that lexicographic
  order. Block b covers keys [b*B, min((b+1)*B, n_s)).
* Cost: q_s * len_b * heads, where heads is the number of query heads the unit
  serves (g = Hq/Hkv for a per-KV-head unit; Hq when a unit is a whole
  (sequence, block) pair, the coarser granularity). Integer arithmetic.
* Roofline-aware cost (an alternative the pages do not give; their cost counts
  query rows only, so a block read for a single query row looks nearly free):
  with a ridge of R query rows per KV head, a unit costs len_b * max(q_s * g, R)
  for each KV head it covers. Its block is streamed in time proportional to len_b
  whatever the rows, and its scores take time proportional to len_b * rows once
  the rows exceed the machine's flop-per-byte ratio, expressed in rows (R). R = 0
  is the pages' cost again.
* LPT (Graham): take units by cost, largest first, ties in enumeration order
  (a stable sort); give each to the worker with the least load so far, ties to the
  lowest worker index. A worker's units are kept in the order they were given.
* Imbalance rate: (max load - mean load) / mean load over all m workers, computed
  as (m * max - total) / total with one float64 division. The KV-Pipe page uses the
  same notion as a max/mean ratio driven toward 1.
"""

from __future__ import annotations

import heapq
import itertools
from typing import Dict, List, Sequence, Tuple

UNIT_SEQ_BLOCK_KVHEAD = 0
UNIT_SEQ_BLOCK = 1


def enumerate_units(
    kv_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    block_len: int,
    granularity: int = UNIT_SEQ_BLOCK_KVHEAD,
    ridge_rows: int = 0,
) -> List[Tuple[int, int, int, int, int]]:
    """Units as (seq, block, kv_head, length, cost); kv_head = -1 for whole-block units.

    ridge_rows = 0 gives the pages' cost, q * length * heads; ridge_rows = R > 0 the
    roofline-aware length * max(q * g, R) per KV head covered."""
    g = num_q_heads // num_kv_heads
    units = []
    for s, (n, q) in enumerate(zip(kv_lens, q_lens)):
        n, q = int(n), int(q)
        nb = -(-n // block_len)
        for b in range(nb):
            length = min(block_len, n - b * block_len)
            if ridge_rows == 0:
                per_kv = q * length * g
            else:
                per_kv = length * max(q * g, ridge_rows)
            if granularity == UNIT_SEQ_BLOCK_KVHEAD:
                for kappa in range(num_kv_heads):
                    units.append((s, b, kappa, length, per_kv))
            else:
                units.append((s, b, -1, length, per_kv * num_kv_heads))
    return units


def lpt_ref(costs: Sequence[int], m: int) -> Tuple[List[int], List[List[int]], List[int]]:
    """Graham's LPT list schedule.

    Returns (worker_of[n], per-worker unit lists in assignment order, loads[m]).
    """
    order = sorted(range(len(costs)), key=lambda u: -costs[u])  # Python's sort is stable
    heap = [(0, w) for w in range(m)]
    worker_of = [-1] * len(costs)
    lists: List[List[int]] = [[] for _ in range(m)]
    loads = [0] * m
    for u in order:
        load, w = heapq.heappop(heap)
        worker_of[u] = w
        lists[w].append(u)
        loads[w] = load + costs[u]
        heapq.heappush(heap, (loads[w], w))
    return worker_of, lists, loads


def imbalance_ref(loads: Sequence[int]) -> float:
    """(max - mean) / mean of the worker loads, as (m*max - total) / total."""
    total = sum(loads)
    if total == 0:
        return 0.0
    return float(len(loads) * max(loads) - total) / float(total)


def plan_ref(
    kv_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    block_len: int,
    num_workers: int,
    granularity: int = UNIT_SEQ_BLOCK_KVHEAD,
    ridge_rows: int = 0,
) -> Dict[str, object]:
    """The whole plan: units, assignment, CSR lists, loads, makespan and imbalance."""
    units = enumerate_units(kv_lens, q_lens, num_q_heads, num_kv_heads, block_len, granularity, ridge_rows)
    costs = [u[4] for u in units]
    worker_of, lists, loads = lpt_ref(costs, num_workers)
    ptr = [0]
    flat: List[int] = []
    for lst in lists:
        flat.extend(lst)
        ptr.append(len(flat))
    total = sum(costs)
    return {
        "units": units,
        "costs": costs,
        "worker_of": worker_of,
        "worker_ptr": ptr,
        "worker_units": flat,
        "loads": loads,
        "makespan": max(loads) if loads else 0,
        "total_cost": total,
        "imbalance": imbalance_ref(loads),
    }


def opt_exhaustive(costs: Sequence[int], m: int) -> int:
    """Optimal makespan by trying every assignment (first unit pinned to worker 0,
    which loses nothing since workers are interchangeable). For tiny instances."""
    n = len(costs)
    if n == 0:
        return 0
    best = None
    for rest in itertools.product(range(m), repeat=n - 1):
        loads = [0] * m
        loads[0] = costs[0]
        for u, w in enumerate(rest, start=1):
            loads[w] += costs[u]
        mk = max(loads)
        if best is None or mk < best:
            best = mk
    return best
