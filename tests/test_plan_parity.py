"""The library's C++ LPT planner against the pure-Python oracle, bit for bit (CPU)."""

import numpy as np
import pytest

from oracle import plan_ref
import split_kv_exact_amd as skv
from split_kv_exact_amd import splitkv_plan
from workloads import WORKLOADS, get_workload


def compare(kv, q, hq, hkv, b, m, gran=0, d=128, ridge=0):
    pl = splitkv_plan(kv, q, hq, hkv, d, b, m, True, gran, ridge)
    ex = pl.export()
    inf = pl.info()
    ref = plan_ref(kv, q, hq, hkv, b, m, gran, ridge)
    units = ref["units"]
    assert inf["num_units"] == len(units)
    assert ex["unit_seq"].tolist() == [u[0] for u in units]
    assert ex["unit_block"].tolist() == [u[1] for u in units]
    assert ex["unit_kv_head"].tolist() == [u[2] for u in units]
    assert ex["unit_len"].tolist() == [u[3] for u in units]
    assert ex["unit_cost"].tolist() == ref["costs"]
    assert ex["worker_of"].tolist() == ref["worker_of"]
    assert ex["worker_ptr"].tolist() == ref["worker_ptr"]
    assert ex["worker_units"].tolist() == ref["worker_units"]
    assert ex["load"].tolist() == ref["loads"]
    assert inf["makespan"] == ref["makespan"]
    assert inf["total_cost"] == ref["total_cost"]
    assert inf["imbalance"] == ref["imbalance"]  # the same float64 division, bit for bit
    costs = ref["costs"]
    assert inf["lower_bound"] == max(-(-sum(costs) // m), max(costs))
    return inf


@pytest.mark.parametrize("key", sorted(WORKLOADS))
@pytest.mark.parametrize("gran", [0, 1])
@pytest.mark.parametrize("ridge", [0, 128, 312])
def test_workload_plans_bit_exact(key, gran, ridge):
    wl = get_workload(key)
    compare(wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.block_len, wl.num_workers, gran,
            wl.head_dim, ridge)


def test_random_instances_bit_exact():
    rng = np.random.default_rng(30)
    for _ in range(40):
        S = int(rng.integers(1, 12))
        hkv = int(rng.integers(1, 5))
        g = int(rng.integers(1, 5))
        b = int(rng.choice([1, 3, 16, 100, 512]))
        m = int(rng.integers(1, 40))
        kv = [int(x) for x in rng.integers(1, 3000, size=S)]
        q = [int(rng.integers(1, k + 1)) for k in kv]
        q = [min(x, 50) for x in q]
        compare(kv, q, g * hkv, hkv, b, m, int(rng.integers(0, 2)), ridge=int(rng.choice([0, 1, 7, 128])))


def test_worker_count_larger_than_units():
    inf = compare([10], [2], 2, 1, 4, 64)
    assert inf["makespan"] == inf["lower_bound"]


def test_xcd_speeds_leave_the_plan_unchanged():
    """Speeds only place workers on workgroups: the exported LPT plan is identical."""
    wl = get_workload("batch8")
    a = skv_plan(wl, None)
    b = skv_plan(wl, [1000, 920, 1000, 980, 1000, 920, 1000, 980])
    for key in a:
        assert np.array_equal(a[key], b[key]), key


def skv_plan(wl, speeds):
    from split_kv_exact_amd import plan_for
    return plan_for(wl, 0, speeds).export()


def test_executed_schedule_balance():
    """The plan info's modelled balance of the schedules as they run. When every unit is
    one job (at most 256 query rows per KV head) the static lists are the plan's worker
    lists, so under the page's cost their imbalance is the plan's, bit for bit; the
    job-time estimate and the simulated queue give non-negative figures."""
    for key in ("batch8", "decode", "lognormal", "mixed", "long"):
        wl = get_workload(key)
        inf = skv.plan_for(wl).info()
        assert inf["num_jobs"] >= inf["num_units"]
        for f in ("exec_imbalance_static", "exec_imbalance_static_est", "exec_imbalance_queue_est"):
            assert inf[f] >= 0.0, (key, f)
        if inf["num_jobs"] == inf["num_units"]:
            assert inf["exec_imbalance_static"] == inf["imbalance"], key
        assert inf["auto_schedule"] in (1, 2)
    # 2048 equal units on 256 workers (two row passes each): every schedule balanced.
    inf = skv.plan_for(get_workload("long")).info()
    assert inf["exec_imbalance_static"] == 0.0 and inf["exec_imbalance_queue_est"] == 0.0
