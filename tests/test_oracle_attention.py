"""Pins for the float64 attention oracle (CPU only).

Each test checks the oracle against something other than itself: a closed form, an
invariant of softmax attention, 50-digit brute force, or torch's own attention
routine. Readings taken where the pages are silent (bottom-right causal alignment,
1/sqrt(D) scale, contiguous GQA groups, natural-log LSE) are pinned here too.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attend_rows, attention_ref, merge_ref, partials_ref, sample_ref


def _rand_problem(rng, kv_lens, q_lens, hq, hkv, d):
    q = rng.standard_normal((sum(q_lens), hq, d))
    k = rng.standard_normal((sum(kv_lens), hkv, d))
    v = rng.standard_normal((sum(kv_lens), hkv, d))
    return q, k, v


def _offs(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(int)


@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_give_mean_of_visible_values(causal):
    # q = 0 makes every score 0, so the softmax is uniform over the visible keys:
    # O_i = mean of visible V rows and LSE_i = ln(#visible).
    rng = np.random.default_rng(1)
    kv_lens, q_lens, hq, hkv, d = [37, 11], [5, 11], 4, 2, 8
    q, k, v = _rand_problem(rng, kv_lens, q_lens, hq, hkv, d)
    q[:] = 0.0
    O, L = attention_ref(q, k, v, kv_lens, q_lens, hq, hkv, causal=causal)
    qo, ko = _offs(q_lens), _offs(kv_lens)
    g = hq // hkv
    for s, (n, qs) in enumerate(zip(kv_lens, q_lens)):
        for i in range(qs):
            nvis = (n - qs + i + 1) if causal else n
            for h in range(hq):
                vs = v[ko[s]:ko[s] + nvis, h // g]
                np.testing.assert_allclose(O[qo[s] + i, h], vs.mean(axis=0), rtol=0, atol=1e-14)
                assert abs(L[qo[s] + i, h] - math.log(nvis)) < 1e-14


def test_causal_alignment_closed_form():
    # q = 0 and v_j = (j mod 2) in every component: row i at position p_i sees keys
    # 0..p_i, of which floor((p_i+1)/2) are odd, so O_i = floor((p_i+1)/2)/(p_i+1).
    # Top-left alignment (p_i = i) would give a different value for every row.
    n, qs, d = 50, 7, 4
    q = np.zeros((qs, 1, d))
    k = np.random.default_rng(2).standard_normal((n, 1, d))
    v = np.repeat((np.arange(n) % 2).astype(float)[:, None, None], d, axis=2)
    O, _ = attention_ref(q, k, v, [n], [qs], 1, 1, causal=True)
    for i in range(qs):
        p = n - qs + i
        expect = ((p + 1) // 2) / (p + 1)
        np.testing.assert_allclose(O[i, 0], expect, rtol=0, atol=1e-15)
        top_left = ((i + 1) // 2) / (i + 1)
        assert abs(O[i, 0, 0] - top_left) > 1e-3


def test_constant_values_are_reproduced():
    rng = np.random.default_rng(3)
    kv_lens, q_lens, hq, hkv, d = [64, 9], [3, 9], 6, 3, 16
    q, k, v = _rand_problem(rng, kv_lens, q_lens, hq, hkv, d)
    c = rng.standard_normal((hkv, d))
    v[:] = c[None]
    O, _ = attention_ref(q, k, v, kv_lens, q_lens, hq, hkv)
    for h in range(hq):
        np.testing.assert_allclose(O[:, h], np.broadcast_to(c[h // 2], O[:, h].shape), rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    # A key aligned with the query and 60x longer dominates every other score by a
    # margin of hundreds: O equals that key's value to rounding.
    rng = np.random.default_rng(4)
    n, d = 40, 8
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((n, 1, d))
    v = rng.standard_normal((n, 1, d))
    j = 17
    k[j, 0] = 60.0 * q[0, 0]
    O, L = attention_ref(q, k, v, [n], [1], 1, 1, causal=True)
    np.testing.assert_allclose(O[0, 0], v[j, 0], rtol=0, atol=1e-12)
    s_j = 60.0 * float(q[0, 0] @ q[0, 0]) / math.sqrt(d)
    assert abs(L[0, 0] - s_j) < 1e-9


def test_mpmath_bruteforce_tiny():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 50
    rng = np.random.default_rng(5)
    for trial in range(6):
        n = int(rng.integers(1, 65))
        qs = int(rng.integers(1, min(4, n) + 1))
        d = int(rng.integers(1, 9))
        g = int(rng.integers(1, 3))
        hkv = int(rng.integers(1, 3))
        hq = g * hkv
        causal = bool(trial % 2 == 0)
        q, k, v = _rand_problem(rng, [n], [qs], hq, hkv, d)
        scale = 1.0 / math.sqrt(d)
        O, L = attention_ref(q, k, v, [n], [qs], hq, hkv, causal=causal)
        for i in range(qs):
            p = n - qs + i
            nvis = p + 1 if causal else n
            for h in range(hq):
                kap = h // g
                w = []
                for j in range(nvis):
                    s = mpmath.mpf(0)
                    for dd in range(d):
                        s += mpmath.mpf(q[i, h, dd]) * mpmath.mpf(k[j, kap, dd])
                    w.append(mpmath.exp(s * mpmath.mpf(scale)))
                tot = mpmath.fsum(w)
                for dd in range(d):
                    o = mpmath.fsum(w[j] * mpmath.mpf(v[j, kap, dd]) for j in range(nvis)) / tot
                    assert abs(float(o) - O[i, h, dd]) <= 1e-13 * max(1.0, abs(float(o)))
                assert abs(float(mpmath.log(tot)) - L[i, h]) <= 1e-13 * max(1.0, abs(float(mpmath.log(tot))))


@pytest.mark.parametrize("causal", [True, False])
def test_matches_torch_sdpa_float64(causal):
    # torch's attention on the CPU in float64, with an explicit bottom-right boolean
    # mask (its is_causal flag is top-left aligned when q != n) and the GQA heads
    # expanded explicitly; LSE from torch.logsumexp of the masked scores.
    rng = np.random.default_rng(6)
    kv_lens, q_lens, hq, hkv, d = [300, 77, 129], [16, 1, 33], 8, 2, 32
    q, k, v = _rand_problem(rng, kv_lens, q_lens, hq, hkv, d)
    O, L = attention_ref(q, k, v, kv_lens, q_lens, hq, hkv, causal=causal)
    qo, ko = _offs(q_lens), _offs(kv_lens)
    g = hq // hkv
    for s, (n, qs) in enumerate(zip(kv_lens, q_lens)):
        Q = torch.from_numpy(q[qo[s]:qo[s + 1]]).permute(1, 0, 2)  # [Hq, q, D]
        K = torch.from_numpy(k[ko[s]:ko[s + 1]]).permute(1, 0, 2).repeat_interleave(g, dim=0)
        V = torch.from_numpy(v[ko[s]:ko[s + 1]]).permute(1, 0, 2).repeat_interleave(g, dim=0)
        pos = torch.arange(n - qs, n)[:, None]
        mask = (torch.arange(n)[None, :] <= pos) if causal else torch.ones(qs, n, dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask)
        np.testing.assert_allclose(O[qo[s]:qo[s + 1]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        scores = (Q @ K.transpose(1, 2)) / math.sqrt(d)
        scores = scores.masked_fill(~mask, float("-inf"))
        lse = torch.logsumexp(scores, dim=-1).permute(1, 0).numpy()
        np.testing.assert_allclose(L[qo[s]:qo[s + 1]], lse, rtol=0, atol=1e-12)


def test_split_invariance_random_partitions():
    # Any partition of a row's keys, each part reduced to (O_b, LSE_b) and merged by
    # log-sum-exp, reproduces the unsplit result (exactness, Split-KV page).
    rng = np.random.default_rng(7)
    for trial in range(20):
        n = int(rng.integers(1, 400))
        qs = int(rng.integers(1, min(n, 40) + 1))
        d = int(rng.choice([4, 16, 64]))
        causal = bool(rng.integers(0, 2))
        Q = rng.standard_normal((qs, d)) * (3.0 if trial % 3 == 0 else 1.0)
        K = rng.standard_normal((n, d))
        V = rng.standard_normal((n, d))
        pos = np.arange(n - qs, n)
        sc = 1.0 / math.sqrt(d)
        O, L = attend_rows(Q, pos, K, V, sc, causal)
        ncut = int(rng.integers(0, min(n, 12)))
        cuts = sorted(set(int(c) for c in rng.integers(1, max(2, n), size=ncut)))
        edges = [0] + [c for c in cuts if 0 < c < n] + [n]
        parts = [attend_rows(Q, pos, K, V, sc, causal, a, b) for a, b in zip(edges[:-1], edges[1:])]
        Om, Lm = merge_ref(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
        np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Lm, L, rtol=1e-12, atol=1e-13)
        # Block size 1: every key its own partial.
        if n <= 120:
            parts = [attend_rows(Q, pos, K, V, sc, causal, j, j + 1) for j in range(n)]
            Om, Lm = merge_ref(np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
            np.testing.assert_allclose(Om, O, rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(Lm, L, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("block_len", [1, 7, 64, 100, 1000])
def test_block_partials_merge_to_full(block_len):
    rng = np.random.default_rng(8)
    kv_lens, q_lens, hq, hkv, d = [130, 64, 5], [9, 64, 2], 4, 2, 16
    q, k, v = _rand_problem(rng, kv_lens, q_lens, hq, hkv, d)
    O, L = attention_ref(q, k, v, kv_lens, q_lens, hq, hkv)
    parts = partials_ref(q, k, v, kv_lens, q_lens, hq, hkv, block_len)
    qo = _offs(q_lens)
    g = hq // hkv
    for s, n in enumerate(kv_lens):
        nb = -(-n // block_len)
        for kap in range(hkv):
            Ob = np.stack([parts[(s, b, kap)][0] for b in range(nb)])
            Lb = np.stack([parts[(s, b, kap)][1] for b in range(nb)])
            Om, Lm = merge_ref(Ob, Lb)
            np.testing.assert_allclose(Om, O[qo[s]:qo[s + 1], kap * g:(kap + 1) * g], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(Lm, L[qo[s]:qo[s + 1], kap * g:(kap + 1) * g], rtol=1e-12, atol=1e-13)


def test_partials_empty_rows_are_minus_inf():
    # Under the causal mask, a block that starts after a row's position has no
    # visible key for that row: its partial is (0, -inf).
    rng = np.random.default_rng(9)
    n, qs, d, B = 20, 6, 4, 4
    q, k, v = _rand_problem(rng, [n], [qs], 1, 1, d)
    parts = partials_ref(q, k, v, [n], [qs], 1, 1, B)
    O4, L4 = parts[(0, 4, 0)]  # keys 16..19
    for i in range(qs):
        p = n - qs + i  # 14..19
        if p < 16:
            assert L4[i, 0] == -np.inf and np.all(O4[i, 0] == 0.0)
        else:
            assert np.isfinite(L4[i, 0])


def test_merge_identity_and_order_invariance():
    rng = np.random.default_rng(10)
    nb, r, d = 6, 5, 8
    Ob = rng.standard_normal((nb, r, d))
    Lb = rng.standard_normal((nb, r)) * 4
    Om, Lm = merge_ref(Ob, Lb)
    # An empty partial (LSE = -inf) changes nothing, whatever its O holds.
    Oe = np.concatenate([Ob, rng.standard_normal((1, r, d))])
    Le = np.concatenate([Lb, np.full((1, r), -np.inf)])
    Om2, Lm2 = merge_ref(Oe, Le)
    np.testing.assert_allclose(Om2, Om, rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(Lm2, Lm, rtol=1e-15, atol=1e-15)
    perm = rng.permutation(nb)
    Om3, Lm3 = merge_ref(Ob[perm], Lb[perm])
    np.testing.assert_allclose(Om3, Om, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(Lm3, Lm, rtol=1e-14, atol=1e-14)
    # Merging in two stages equals merging at once (associativity).
    Oa, La = merge_ref(Ob[:2], Lb[:2])
    Oc, Lc = merge_ref(Ob[2:], Lb[2:])
    Om4, Lm4 = merge_ref(np.stack([Oa, Oc]), np.stack([La, Lc]))
    np.testing.assert_allclose(Om4, Om, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(Lm4, Lm, rtol=1e-14, atol=1e-14)
    # Two partials with equal LSE merge to their mean and LSE + ln 2.
    Om5, Lm5 = merge_ref(np.stack([Ob[0], Ob[1]]), np.stack([Lb[0], Lb[0]]))
    np.testing.assert_allclose(Om5, 0.5 * (Ob[0] + Ob[1]), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(Lm5, Lb[0] + math.log(2.0), rtol=1e-15, atol=1e-15)


def test_sample_ref_matches_full():
    rng = np.random.default_rng(11)
    n, qs, hq, hkv, d = 257, 12, 8, 2, 16
    q, k, v = _rand_problem(rng, [n], [qs], hq, hkv, d)
    O, L = attention_ref(q, k, v, [n], [qs], hq, hkv)
    pairs = [(0, 0), (11, 7), (5, 3), (5, 4), (11, 0)]
    Os, Ls = sample_ref(q, k, v, pairs, hkv)
    for t, (i, h) in enumerate(pairs):
        np.testing.assert_allclose(Os[t], O[i, h], rtol=0, atol=1e-15)
        assert abs(Ls[t] - L[i, h]) < 1e-15


def test_large_scores_do_not_overflow():
    # Scores near +-700 would overflow a naive exp; the max-shifted form must not.
    rng = np.random.default_rng(12)
    n, d = 64, 8
    Q = rng.standard_normal((3, d)) * 60
    K = rng.standard_normal((n, d)) * 60
    V = rng.standard_normal((n, d))
    O, L = attend_rows(Q, np.array([n - 3, n - 2, n - 1]), K, V, 1 / math.sqrt(d), True)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    assert np.all(np.abs(O) <= np.abs(V).max() + 1e-12)
