"""Readers for the text fixtures under tests/golden (no arithmetic of the method)."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_plans(name="lpt_plans.txt"):
    cases, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = cases.setdefault(line.strip("[]"), {})
                continue
            key, val = (x.strip() for x in line.split("=", 1))
            nums = [int(x) for x in val.split()]
            cur[key] = nums if len(nums) != 1 or key in ("kv_lens", "q_lens", "unit_cost", "worker_of",
                                                         "worker_ptr", "worker_units", "loads") else nums[0]
    return cases


def read_graham(name="graham_tight.txt"):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            m, jobs, lpt, opt = (x.strip() for x in line.split("|"))
            rows.append((int(m), [int(x) for x in jobs.split()], int(lpt), int(opt)))
    return rows
