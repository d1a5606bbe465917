"""Strided inputs: Q, K, V and dO given as views with token and head strides other than
the packed ones (K and V interleaved in one KV cache [tokens, 2, Hkv, D]; Q and dO with
padding heads) give the same bits as the packed tensors, forward and backward.

The kernels read Q, K, V and dO through the caller's strides; every other value they
compute is the same, so the outputs must not change by a bit. The cases cover both
forward launches (matrix-path jobs of 8 or more row tiles, streaming jobs) and the
three backward paths (few-row jobs, the dQ pass, the dK/dV key tiles).
"""

import pytest
import torch

import split_kv_exact_amd as skv
from tests.parity import say
from workloads import Workload, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


CASES = [
    Workload(name="strided_mixed_rows", dtype="bfloat16", kv_lens=(3000, 333, 77, 2100, 16), q_lens=(40, 5, 1, 16, 16),
             num_q_heads=32, num_kv_heads=8, head_dim=128, block_len=512, num_workers=16, causal=True, seed=17),
    Workload(name="strided_d64", dtype="bfloat16", kv_lens=(1000, 513), q_lens=(3, 9), num_q_heads=8,
             num_kv_heads=2, head_dim=64, block_len=128, num_workers=7, causal=True, seed=18),
    # fp32 inputs (forward only: the backward pass takes bf16 inputs).
    Workload(name="strided_fp32", dtype="float32", kv_lens=(2048, 300), q_lens=(4, 7), num_q_heads=4,
             num_kv_heads=2, head_dim=64, block_len=256, num_workers=8, causal=True, seed=19),
]


def _strided_copy_kv(k, v):
    """K and V inside one [tokens, 2, Hkv, D] cache: token stride 2 Hkv D, head stride D."""
    cache = torch.empty((k.shape[0], 2) + tuple(k.shape[1:]), dtype=k.dtype, device=k.device)
    cache[:, 0] = k
    cache[:, 1] = v
    return cache[:, 0], cache[:, 1]


def _strided_copy_rows(x, pad_heads=3):
    """x inside a [tokens, H + pad, D] buffer (token stride (H + pad) D)."""
    buf = torch.zeros((x.shape[0], x.shape[1] + pad_heads, x.shape[2]), dtype=x.dtype, device=x.device)
    buf[:, :x.shape[1]] = x
    return buf[:, :x.shape[1]]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_strided_inputs_give_the_packed_results(wl):
    say(f"[gpu] strided inputs {wl.name}")
    q, k, v = make_qkv(wl, "cuda")
    ks, vs = _strided_copy_kv(k, v)
    qs = _strided_copy_rows(q)
    assert not ks.is_contiguous() and not qs.is_contiguous()
    assert ks.stride(0) == 2 * wl.num_kv_heads * wl.head_dim and qs.stride(0) == (wl.num_q_heads + 3) * wl.head_dim
    plan = skv.plan_for(wl)
    dev_plan = skv.splitkv_plan_upload(plan)
    out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v)
    out_s, lse_s = skv.splitkv_attn(plan, dev_plan, qs, ks, vs)
    torch.cuda.synchronize()
    assert torch.equal(out, out_s) and torch.equal(lse, lse_s)
    if wl.dtype != "bfloat16":
        return

    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    do = torch.randn(q.shape, generator=gen, device="cuda", dtype=torch.float32).to(q.dtype)
    dos = _strided_copy_rows(do, pad_heads=1)
    for dt in (torch.float32, torch.bfloat16):
        ref = skv.splitkv_attn_backward(plan, dev_plan, q, k, v, do, out, lse, dkv_dtype=dt)
        got = skv.splitkv_attn_backward(plan, dev_plan, qs, ks, vs, dos, out, lse, dkv_dtype=dt)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), ref, got):
            assert torch.equal(a, b), (name, dt)
