"""Fused steps captured in a HIP graph replay to the eager result, bit for bit.

A caller may capture splitkv_attn in a graph: the library enqueues only kernels (no
memsets, no allocation). Each replay here is checked against the eager call, with eager
steps and synchronisations between replays, under the static and the queue schedules
(the queue's counters live in the plan buffer and are reset by the kernel itself, so a
replay starts from zero like an eager launch).
"""

import pytest
import torch

import split_kv_exact_amd as skv
from tests.parity import say
from workloads import Workload, get_workload, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


CASES = [
    Workload(name="ragged_bf16_d128", dtype="bfloat16", kv_lens=(1000, 333, 77, 2100, 16), q_lens=(16, 5, 1, 40, 16),
             num_q_heads=32, num_kv_heads=8, head_dim=128, block_len=256, num_workers=16, causal=True, seed=7,
             boost_frac=0.0, boost=8.0, granularity=0),
    get_workload("batch8"),
]


@pytest.mark.parametrize("sched", ["static", "queue", "auto"])
@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_graph_replays_match_eager(wl, sched):
    say(f"[gpu] graph replay {wl.name} {sched}")
    q, k, v = make_qkv(wl, "cuda")
    plan = skv.plan_for(wl)
    dev_plan = skv.splitkv_plan_upload(plan)
    ws = skv.workspace(plan)
    out = torch.empty((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((wl.total_q, wl.num_q_heads), dtype=torch.float32, device="cuda")
    skv.splitkv_attn(plan, dev_plan, q, k, v, ws, out, lse, schedule=sched)
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(3):
                skv.splitkv_attn(plan, dev_plan, q, k, v, ws, out, lse, schedule=sched, stream=side)
    torch.cuda.synchronize()
    for r in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"replay {r}"
        skv.splitkv_attn(plan, dev_plan, q, k, v, ws, out, lse, schedule=sched)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), f"eager step after replay {r}"
    assert int(dev_plan[-1024:].count_nonzero()) == 0, "scheduling area not left zero"
    del graph


@pytest.mark.parametrize("dkv", ["float32", "bfloat16"])
@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_backward_graph_replays_match_eager(wl, dkv):
    """splitkv_attn_backward captured in a graph (up to five kernel launches, no memset)
    replays to the eager gradients bit for bit. The ragged case has jobs of all three
    backward paths (few-row jobs, 8-wave dQ workgroups, dK/dV key tiles)."""
    say(f"[gpu] backward graph replay {wl.name} {dkv} dK/dV")
    q, k, v = make_qkv(wl, "cuda")
    plan = skv.plan_for(wl)
    dev_plan = skv.splitkv_plan_upload(plan)
    ws = skv.workspace(plan)
    out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v, ws)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(99)
    do = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype)
    dt = getattr(torch, dkv)
    dq = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dk = torch.empty(k.shape, dtype=dt, device="cuda")
    dv = torch.empty(v.shape, dtype=dt, device="cuda")
    skv.splitkv_attn_backward(plan, dev_plan, q, k, v, do, out, lse, ws, dq, dk, dv)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (dq, dk, dv)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(2):
                skv.splitkv_attn_backward(plan, dev_plan, q, k, v, do, out, lse, ws, dq, dk, dv, stream=side)
    torch.cuda.synchronize()
    for r in range(3):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip((dq, dk, dv), ref)), f"replay {r}"
        skv.splitkv_attn_backward(plan, dev_plan, q, k, v, do, out, lse, ws, dq, dk, dv)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip((dq, dk, dv), ref)), f"eager call after replay {r}"
    del graph
