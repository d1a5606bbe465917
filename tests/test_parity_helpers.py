"""CPU checks of the whole-tensor backward comparison used by the GPU parity tests.

The helper streams per sequence, KV head and key range; here it is fed the oracle's own
whole-batch gradients (so every error must vanish) and the same with one planted
element changed (which it must report), on a ragged causal batch whose key ranges
split sequences unevenly.
"""

import numpy as np
import torch

from oracle import attention_ref
from oracle.backward import attention_grad_ref
from tests.parity import compare_grads_whole
from workloads import Workload, make_qkv, widen_to_f64


def _case():
    wl = Workload(name="helper", dtype="bfloat16", kv_lens=(300, 77, 5), q_lens=(6, 3, 5), num_q_heads=8,
                  num_kv_heads=2, head_dim=64, block_len=64, num_workers=4, seed=3)
    q, k, v = make_qkv(wl, "cpu")
    gen = torch.Generator().manual_seed(4)
    do = torch.randn(q.shape, generator=gen).to(torch.bfloat16)
    O, L = attention_ref(widen_to_f64(q), widen_to_f64(k), widen_to_f64(v), wl.kv_lens, wl.q_lens,
                         wl.num_q_heads, wl.num_kv_heads, wl.causal)
    gq, gk, gv = attention_grad_ref(widen_to_f64(q), widen_to_f64(k), widen_to_f64(v), widen_to_f64(do),
                                    wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.causal, o=O, lse=L)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    return wl, q, k, v, do, t(O), t(L), t(gq), t(gk), t(gv)


def test_whole_backward_comparison_of_the_oracle_with_itself():
    wl, q, k, v, do, O, L, gq, gk, gv = _case()
    res = compare_grads_whole(wl, q, k, v, do, O, L, gq, gk, gv, keys_per_task=50, threads=3)
    for name in ("dq", "dk", "dv"):
        l2, mx = res.errors(name)
        assert l2 < 1e-12 and mx < 1e-12, (name, l2, mx)


def test_whole_backward_comparison_finds_a_planted_error():
    wl, q, k, v, do, O, L, gq, gk, gv = _case()
    gk = gk.clone()
    gk[301, 1, 7] += 0.5  # sequence 1, key 1, KV head 1
    res = compare_grads_whole(wl, q, k, v, do, O, L, gq, gk, gv, keys_per_task=50, threads=3)
    assert res.errors("dk")[1] > 1e-3
    assert res.errors("dq")[0] < 1e-12 and res.errors("dv")[0] < 1e-12
