"""The float64 backward oracle against things other than itself (CPU only).

Pins: central finite differences of the forward oracle (an independent derivative of
the pinned forward), closed forms (zero upstream gradient; identical value rows, where
the output cannot depend on the scores), split invariance (block-wise dQ parts summed
equal the unsplit gradient), and agreement of the sampled form with the whole one.
"""

import numpy as np
import pytest

from oracle import attention_ref
from oracle.backward import attention_grad_ref, grad_sample_ref


def _case(seed, kv, ql, hq, hkv, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((sum(ql), hq, d))
    k = rng.standard_normal((sum(kv), hkv, d))
    v = rng.standard_normal((sum(kv), hkv, d))
    do = rng.standard_normal((sum(ql), hq, d))
    return q, k, v, do


@pytest.mark.parametrize("causal", [True, False])
def test_finite_differences(causal):
    kv, ql, hq, hkv, d = [7, 5], [3, 2], 4, 2, 8
    q, k, v, do = _case(3, kv, ql, hq, hkv, d)

    def loss(q_, k_, v_):
        o, _ = attention_ref(q_, k_, v_, kv, ql, hq, hkv, causal)
        return float((o * do).sum())

    dq, dk, dv = attention_grad_ref(q, k, v, do, kv, ql, hq, hkv, causal)
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            keep = arr[idx]
            arr[idx] = keep + eps
            up = loss(q, k, v)
            arr[idx] = keep - eps
            dn = loss(q, k, v)
            arr[idx] = keep
            num[idx] = (up - dn) / (2 * eps)
        assert np.abs(num - grad).max() <= 1e-6 * max(1.0, np.abs(grad).max())


def test_zero_upstream_gradient():
    kv, ql = [9], [4]
    q, k, v, do = _case(5, kv, ql, 2, 1, 8)
    dq, dk, dv = attention_grad_ref(q, k, v, np.zeros_like(do), kv, ql, 2, 1)
    assert not dq.any() and not dk.any() and not dv.any()


def test_identical_values_closed_form():
    """All value rows equal c: O_i = c whatever the scores, so dQ = dK = 0, and
    dV_j = sum_i P_ij dO_i sums to sum_i dO_i over the keys (each row's P sums to 1)."""
    kv, ql, hq, hkv, d = [11, 6], [4, 3], 4, 2, 8
    q, k, v, do = _case(7, kv, ql, hq, hkv, d)
    v[:] = np.linspace(-1.0, 2.0, d)[None, None, :]
    dq, dk, dv = attention_grad_ref(q, k, v, do, kv, ql, hq, hkv, True)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    g = hq // hkv
    qo, ko = np.cumsum([0] + ql), np.cumsum([0] + kv)
    for s in range(len(kv)):
        for kappa in range(hkv):
            want = do[qo[s]:qo[s + 1], kappa * g:(kappa + 1) * g].sum(axis=(0, 1))
            got = dv[ko[s]:ko[s + 1], kappa].sum(axis=0)
            assert np.allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("block_len", [1, 3, 4, 100])
def test_split_invariance(block_len):
    kv, ql, hq, hkv, d = [13, 4, 9], [5, 4, 1], 6, 3, 8
    q, k, v, do = _case(11, kv, ql, hq, hkv, d)
    whole = attention_grad_ref(q, k, v, do, kv, ql, hq, hkv, True)
    split = attention_grad_ref(q, k, v, do, kv, ql, hq, hkv, True, block_len=block_len)
    for a, b in zip(whole, split):
        assert np.abs(a - b).max() < 1e-12


def test_given_forward_outputs_and_sampled_form():
    kv, ql, hq, hkv, d = [21, 8], [6, 3], 4, 2, 16
    q, k, v, do = _case(13, kv, ql, hq, hkv, d)
    o, lse = attention_ref(q, k, v, kv, ql, hq, hkv, True)
    a = attention_grad_ref(q, k, v, do, kv, ql, hq, hkv, True)
    b = attention_grad_ref(q, k, v, do, kv, ql, hq, hkv, True, o=o, lse=lse)
    for x, y in zip(a, b):
        assert np.abs(x - y).max() < 1e-12
    s, q0, k0 = 0, 0, 0
    pairs = [(0, 0), (5, 3), (2, 1)]
    keys = [(0, 0), (20, 1), (14, 0)]
    dq, dk, dv = grad_sample_ref(q[q0:q0 + 6], k[k0:k0 + 21], v[k0:k0 + 21], do[q0:q0 + 6], o[q0:q0 + 6],
                                 lse[q0:q0 + 6], hkv, pairs, keys)
    for t, (i, h) in enumerate(pairs):
        assert np.abs(dq[t] - a[0][i, h]).max() < 1e-12
    for t, (j, kappa) in enumerate(keys):
        assert np.abs(dk[t] - a[1][j, kappa]).max() < 1e-12
        assert np.abs(dv[t] - a[2][j, kappa]).max() < 1e-12
