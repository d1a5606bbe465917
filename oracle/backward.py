"""float64 gradients of softmax attention, whole and per KV block.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The Split-KV page's setting is training over long contexts, and its claim is that the
sharded computation equals the unsharded one; for the backward pass that means the
gradients too. The pages print no backward formulas, so the definitions here are the
textbook ones for O = softmax(scale * Q K^T + mask) V, with the forward readings of
``oracle.attention`` (bottom-right causal mask, GQA head grouping, natural-log LSE):

For a query row i with visible keys J_i, scores s_ij = scale <q_i, k_j>, probabilities
P_ij = exp(s_ij - LSE_i) and an upstream gradient dO_i:

    D_i   = <dO_i, O_i>                     (= sum_j P_ij <dO_i, v_j>)
    dP_ij = <dO_i, v_j>
    dS_ij = P_ij (dP_ij - D_i)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i         (over the rows of every head of the group)
    dV_j  = sum_i P_ij dO_i

P uses the row's full LSE, so every term involves one key block only: a block's keys
get their dK, dV from that block alone, and dQ_i is the plain sum over blocks of the
block's dQ part. That is the exact split form (tested against the unsplit one).

The functions take the forward outputs O and LSE as inputs (by default computed here
in float64), so that a device backward can be checked on the forward results it was
given; with the float64 forward they are the exact gradients (pinned by central finite
differences of ``oracle.attention.attend_rows`` in the tests).
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .attention import _group_rows, _offsets, attend_rows

_CHUNK_ELEMS = 1 << 22


def grad_rows(
    Q: np.ndarray,
    pos: np.ndarray,
    K: np.ndarray,
    V: np.ndarray,
    dO: np.ndarray,
    O: np.ndarray,
    LSE: np.ndarray,
    scale: float,
    causal: bool,
    key_lo: int = 0,
    key_hi: int | None = None,
) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradient terms of query rows against keys [key_lo, key_hi) of one KV head.

    Q, dO, O: [r, D]; pos: [r] positions; K, V: [n, D]; LSE: [r] full-row log-sum-exp.
    Returns (dQ part [r, D], dK [hi - lo, D], dV [hi - lo, D]), float64.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    LSE = np.asarray(LSE, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    r, d = Q.shape
    n = K.shape[0]
    lo = max(0, int(key_lo))
    hi = n if key_hi is None else min(int(key_hi), n)
    dQ = np.zeros((r, d), dtype=np.float64)
    dK = np.zeros((max(hi - lo, 0), d), dtype=np.float64)
    dV = np.zeros((max(hi - lo, 0), d), dtype=np.float64)
    if r == 0 or hi <= lo:
        return dQ, dK, dV
    Dv = (dO * O).sum(axis=1)  # D_i
    seen = np.isfinite(LSE)
    Lsafe = np.where(seen, LSE, 0.0)
    chunk = max(1, _CHUNK_ELEMS // max(1, r))
    for j0 in range(lo, hi, chunk):
        j1 = min(hi, j0 + chunk)
        s = (Q @ K[j0:j1].T) * scale
        if causal:
            keys = np.arange(j0, j1, dtype=np.int64)
            s[keys[None, :] > pos[:, None]] = -np.inf
        P = np.exp(s - Lsafe[:, None])
        P[~seen] = 0.0
        dP = dO @ V[j0:j1].T
        dS = P * (dP - Dv[:, None])
        dQ += scale * (dS @ K[j0:j1])
        dK[j0 - lo:j1 - lo] = scale * (dS.T @ Q)
        dV[j0 - lo:j1 - lo] = P.T @ dO
    return dQ, dK, dV


def attention_grad_ref(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    do: np.ndarray,
    kv_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    causal: bool = True,
    scale: float | None = None,
    o: np.ndarray | None = None,
    lse: np.ndarray | None = None,
    block_len: int | None = None,
) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of the whole batch.

    q, do: [sum q_s, Hq, D]; k, v: [sum n_s, Hkv, D]; o, lse: the forward outputs
    ([sum q_s, Hq, D], [sum q_s, Hq]; computed here when None). With block_len, dQ is
    summed over the blocks' parts one block at a time (the split form).
    Returns dq [sum q_s, Hq, D], dk and dv [sum n_s, Hkv, D], float64.
    """
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = num_q_heads // num_kv_heads
    qo, ko = _offsets(q_lens), _offsets(kv_lens)
    dq = np.zeros((q.shape[0], num_q_heads, d), dtype=np.float64)
    dk = np.zeros((k.shape[0], num_kv_heads, d), dtype=np.float64)
    dv = np.zeros((k.shape[0], num_kv_heads, d), dtype=np.float64)
    for s, (n, qs) in enumerate(zip(kv_lens, q_lens)):
        pos = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)
        for kappa in range(num_kv_heads):
            rows = _group_rows(q[qo[s]:qo[s + 1]], kappa, g)
            drows = _group_rows(do[qo[s]:qo[s + 1]], kappa, g)
            ks, vs = k[ko[s]:ko[s + 1], kappa], v[ko[s]:ko[s + 1], kappa]
            if o is None or lse is None:
                orows, lrows = attend_rows(rows, pos, ks, vs, sc, causal)
            else:
                orows = _group_rows(o[qo[s]:qo[s + 1]], kappa, g)
                lrows = np.asarray(lse[qo[s]:qo[s + 1], kappa * g:(kappa + 1) * g], dtype=np.float64).reshape(-1)
            bounds = [(0, n)] if block_len is None else [(b, min(b + block_len, n)) for b in range(0, n, block_len)]
            dqr = np.zeros((qs * g, d), dtype=np.float64)
            for lo, hi in bounds:
                dqb, dkb, dvb = grad_rows(rows, pos, ks, vs, drows, orows, lrows, sc, causal, lo, hi)
                dqr += dqb
                dk[ko[s] + lo:ko[s] + hi, kappa] = dkb
                dv[ko[s] + lo:ko[s] + hi, kappa] = dvb
            dq[qo[s]:qo[s + 1], kappa * g:(kappa + 1) * g] = dqr.reshape(qs, g, d)
    return dq, dk, dv


def grad_sample_ref(
    q_seq: np.ndarray,
    k_seq: np.ndarray,
    v_seq: np.ndarray,
    do_seq: np.ndarray,
    o_seq: np.ndarray,
    lse_seq: np.ndarray,
    num_kv_heads: int,
    pairs: List[Tuple[int, int]],
    keys: List[Tuple[int, int]],
    causal: bool = True,
    scale: float | None = None,
) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Selected gradient entries of one sequence, for checks at sizes too large to run
    whole: dQ of (query index i, query head h) pairs, dK and dV of (key j, KV head)
    pairs. o_seq / lse_seq are the forward outputs the gradients are taken at.
    Returns dq [len(pairs), D], dk [len(keys), D], dv [len(keys), D].
    """
    qs, hq, d = q_seq.shape
    n = k_seq.shape[0]
    g = hq // num_kv_heads
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = np.zeros((len(pairs), d), dtype=np.float64)
    for t, (i, h) in enumerate(pairs):
        kappa = h // g
        pos = np.array([n - qs + i], dtype=np.int64)
        dqt, _, _ = grad_rows(q_seq[i:i + 1, h], pos, k_seq[:, kappa], v_seq[:, kappa], do_seq[i:i + 1, h],
                              o_seq[i:i + 1, h], lse_seq[i:i + 1, h], sc, causal)
        dq[t] = dqt[0]
    dk = np.zeros((len(keys), d), dtype=np.float64)
    dv = np.zeros((len(keys), d), dtype=np.float64)
    pos_all = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)
    for t, (j, kappa) in enumerate(keys):
        rows = _group_rows(q_seq, kappa, g)
        drows = _group_rows(do_seq, kappa, g)
        orows = _group_rows(o_seq, kappa, g)
        lrows = np.asarray(lse_seq[:, kappa * g:(kappa + 1) * g], dtype=np.float64).reshape(-1)
        _, dkt, dvt = grad_rows(rows, pos_all, k_seq[:, kappa], v_seq[:, kappa], drows, orows, lrows, sc, causal,
                                j, j + 1)
        dk[t] = dkt[0]
        dv[t] = dvt[0]
    return dq, dk, dv
