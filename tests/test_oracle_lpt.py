"""Pins for the pure-Python LPT planner oracle (CPU only).

Pinned against: Graham's tight family (closed form), Graham's 4/3 - 1/(3m) bound
against brute-force optima on random tiny instances, the n <= m and equal-cost
special cases, and hand-derived golden plans (tests/golden/lpt_plans.txt).
"""

import itertools

import numpy as np
import pytest

from oracle import enumerate_units, imbalance_ref, lpt_ref, opt_exhaustive, plan_ref
from oracle.lpt import UNIT_SEQ_BLOCK, UNIT_SEQ_BLOCK_KVHEAD
from tests.golden_io import read_graham, read_plans
from workloads import get_workload


@pytest.mark.parametrize("row", read_graham())
def test_graham_tight_family(row):
    m, jobs, lpt_mk, opt_mk = row
    _, _, loads = lpt_ref(jobs, m)
    assert max(loads) == lpt_mk == 4 * m - 1
    assert opt_exhaustive(jobs, m) == opt_mk == 3 * m
    # The family attains Graham's bound exactly: LPT/OPT = 4/3 - 1/(3m).
    assert 3 * m * lpt_mk == (4 * m - 1) * opt_mk


def test_graham_bound_on_random_tiny_instances():
    rng = np.random.default_rng(20)
    for _ in range(60):
        m = int(rng.integers(1, 5))
        n = int(rng.integers(1, 9 if m <= 3 else 8))
        costs = [int(c) for c in rng.integers(1, 50, size=n)]
        _, _, loads = lpt_ref(costs, m)
        opt = opt_exhaustive(costs, m)
        lpt = max(loads)
        assert opt <= lpt
        assert 3 * m * lpt <= (4 * m - 1) * opt  # LPT <= (4/3 - 1/(3m)) OPT, in integers
        assert opt >= max(max(costs), -(-sum(costs) // m))


def test_opt_exhaustive_closed_forms():
    assert opt_exhaustive([1] * 7, 3) == 3
    assert opt_exhaustive([3, 3, 2, 2, 2], 2) == 6
    assert opt_exhaustive([10, 1, 1], 2) == 10
    assert opt_exhaustive([4, 4, 4, 4], 4) == 4
    assert opt_exhaustive([5], 3) == 5


def test_few_units_is_optimal():
    rng = np.random.default_rng(21)
    for _ in range(20):
        m = int(rng.integers(1, 9))
        n = int(rng.integers(1, m + 1))
        costs = [int(c) for c in rng.integers(1, 1000, size=n)]
        worker_of, _, loads = lpt_ref(costs, m)
        assert max(loads) == max(costs)
        assert sorted(worker_of) == sorted(set(worker_of))  # one unit per worker


def test_equal_costs_zero_imbalance_long_context_and_small():
    wl = get_workload("long")  # 256 blocks x 8 KV heads = 2048 equal units, 256 workers
    p = plan_ref(wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.block_len, wl.num_workers)
    assert len(p["units"]) == 2048
    assert p["imbalance"] == 0.0 and p["makespan"] * 256 == p["total_cost"]
    wl = get_workload("small")  # 8 blocks on 8 workers
    p = plan_ref(wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.block_len, wl.num_workers)
    assert len(p["units"]) == 8 and p["imbalance"] == 0.0
    assert p["worker_of"] == list(range(8))


@pytest.mark.parametrize("name", sorted(read_plans()))
def test_golden_plans(name):
    c = read_plans()[name]
    p = plan_ref(c["kv_lens"], c["q_lens"], c["num_q_heads"], c["num_kv_heads"], c["block_len"],
                 c["num_workers"], c["granularity"])
    assert p["costs"] == c["unit_cost"]
    assert p["worker_of"] == c["worker_of"]
    assert p["worker_ptr"] == c["worker_ptr"]
    assert p["worker_units"] == c["worker_units"]
    assert p["loads"] == c["loads"]
    assert p["makespan"] == c["makespan"]
    assert p["total_cost"] == c["total_cost"]
    assert p["imbalance"] == c["imbalance_num"] / c["imbalance_den"]


def test_enumeration_ragged_tail():
    units = enumerate_units([1000], [3], 8, 2, 256)
    assert [u[3] for u in units if u[2] == 0] == [256, 256, 256, 232]
    assert [(u[0], u[1], u[2]) for u in units[:4]] == [(0, 0, 0), (0, 0, 1), (0, 1, 0), (0, 1, 1)]
    assert all(u[4] == 3 * u[3] * 4 for u in units)
    whole = enumerate_units([1000], [3], 8, 2, 256, granularity=1)
    assert [u[4] for u in whole] == [3 * 256 * 8] * 3 + [3 * 232 * 8]


def test_imbalance_definition():
    assert imbalance_ref([3, 1]) == 0.5
    assert imbalance_ref([2, 2, 2]) == 0.0
    assert imbalance_ref([0, 0]) == 0.0


def test_every_unit_assigned_once_and_lists_in_assignment_order():
    rng = np.random.default_rng(22)
    costs = [int(c) for c in rng.integers(1, 100, size=200)]
    worker_of, lists, loads = lpt_ref(costs, 7)
    assert sorted(itertools.chain(*lists)) == list(range(200))
    for w, lst in enumerate(lists):
        assert all(worker_of[u] == w for u in lst)
        assert sum(costs[u] for u in lst) == loads[w]
        # a worker receives units in non-increasing cost order (LPT order)
        assert all(costs[a] >= costs[b] for a, b in zip(lst, lst[1:]))


def test_roofline_cost_worked_example():
    """Roofline-aware unit costs, computed by hand.

    Two sequences, Hq = 8 over Hkv = 2 (g = 4), B = 4096, ridge R = 128 rows:
      seq 0: n = 5000, q = 2 -> 8 rows per KV head, blocks of 4096 and 904 keys:
             4096 * max(8, 128) = 524288 and 904 * 128 = 115712 per KV head;
      seq 1: n = 300, q = 40 -> 160 rows, one block: 300 * 160 = 48000 (rows above
             R, so the same as the pages' cost 40 * 300 * 4).
    The pages' costs of seq 0's blocks would be 2 * 4096 * 4 = 32768 and 7232.
    """
    units = enumerate_units([5000, 300], [2, 40], 8, 2, 4096, UNIT_SEQ_BLOCK_KVHEAD, 128)
    assert [u[4] for u in units] == [524288, 524288, 115712, 115712, 48000, 48000]
    assert [u[3] for u in units] == [4096, 4096, 904, 904, 300, 300]
    whole = enumerate_units([5000, 300], [2, 40], 8, 2, 4096, UNIT_SEQ_BLOCK, 128)
    assert [u[4] for u in whole] == [1048576, 231424, 96000]
    pages = enumerate_units([5000, 300], [2, 40], 8, 2, 4096, UNIT_SEQ_BLOCK_KVHEAD, 0)
    assert [u[4] for u in pages] == [32768, 32768, 7232, 7232, 48000, 48000]
    # LPT on two workers: 524288 each, then 115712 each, then 48000 each.
    plan = plan_ref([5000, 300], [2, 40], 8, 2, 4096, 2, UNIT_SEQ_BLOCK_KVHEAD, 128)
    assert plan["loads"] == [688000, 688000]
    assert plan["worker_units"] == [0, 2, 4, 1, 3, 5]
    assert plan["imbalance"] == 0.0
