"""splitkv_attn_scratch (the entry point that allocates nothing) against splitkv_attn.

Both run the same kernels over the same plan; the scratch entry point only swaps the
caller's workspace for the library's own per-GPU array. Two calls in a row, the
second on a smaller problem, must each give splitkv_attn's outputs bit for bit (and
so the oracle's, which the other parity tests compare splitkv_attn with).
"""

import pytest
import torch

import split_kv_exact_amd as skv
from split_kv_exact_amd import _lib as L
from tests.parity import say
from workloads import Workload, get_workload, make_qkv

pytestmark = pytest.mark.gpu


def _small():
    return Workload(name="ragged_bf16_d128", dtype="bfloat16", kv_lens=(1000, 333, 77, 2100, 16),
                    q_lens=(16, 5, 1, 40, 16), num_q_heads=32, num_kv_heads=8, head_dim=128, block_len=256,
                    num_workers=16, seed=7)


def test_scratch_entry_point_matches_splitkv_attn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    results = []
    for wl in (get_workload("batch8"), _small()):
        say(f"[gpu] splitkv_attn_scratch on {wl.name}")
        q, k, v = make_qkv(wl, "cuda")
        plan = skv.plan_for(wl)
        assert plan.info()["workspace_bytes"] <= L.SPLITKV_SCRATCH_BYTES
        dev_plan = skv.splitkv_plan_upload(plan)
        ref_o, ref_l = skv.splitkv_attn(plan, dev_plan, q, k, v)
        out = torch.full_like(ref_o, float("nan"))
        lse = torch.full_like(ref_l, float("nan"))
        skv.splitkv_attn_scratch(plan, dev_plan, q, k, v, out, lse)
        torch.cuda.synchronize()
        same = torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        say(f"  identical to splitkv_attn: {same}")
        results.append(same)
        assert same, wl.name
    assert all(results)


def test_scratch_entry_point_rejects_large_workspaces():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = get_workload("lognormal")  # about 2 GB of partials
    plan = skv.plan_for(wl)
    assert plan.info()["workspace_bytes"] > L.SPLITKV_SCRATCH_BYTES
    dev_plan = skv.splitkv_plan_upload(plan)
    q = torch.zeros((wl.total_q, wl.num_q_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    # K and V of the right shape without their memory (token stride 0): the call must
    # fail on the workspace size before it launches anything.
    k = torch.zeros((1, wl.num_kv_heads, wl.head_dim), dtype=torch.bfloat16, device="cuda").expand(
        wl.total_kv, -1, -1)
    with pytest.raises(skv.SplitKVError) as e:
        skv.splitkv_attn_scratch(plan, dev_plan, q, k, k)
    assert e.value.status == L.SPLITKV_ERR_WORKSPACE
