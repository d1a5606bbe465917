"""float64 softmax attention, per-block partials and the log-sum-exp merge.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Problem (Split-KV page, lede and "Timeline"): a batch of sequences, each with a long
key/value context and a short block of queries; the context is cut into KV blocks,
each block yields a result the size of the queries, and combining those results must
give exactly what unsharded attention gives. The pages print no formulas, so the
definitions below are the textbook ones, with these readings:

* Queries are the last q tokens of an n-token context, so query row i sits at
  position p_i = n - q + i. Under the causal mask it sees keys 0..p_i, itself
  included (bottom-right alignment).
* Scores are scale * <q, k> with scale = 1/sqrt(D) unless given.
* Grouped-query attention: query head h reads KV head floor(h / g), g = Hq / Hkv.
* A row that sees no key of a block has partial output 0 and log-sum-exp -inf.
* Log-sum-exp uses the natural logarithm.

The full result is computed in two passes over key chunks with one global row
maximum per row (pass 1: max; pass 2: sum of exp and weighted values, one division
at the end). Chunking only bounds memory; the merge formula is never used for it,
so comparing merged partials against it is a real test of the merge.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

# Rows x keys per score chunk (float64): 4M entries, 32 MiB.
_CHUNK_ELEMS = 1 << 22


def _offsets(lens: Sequence[int]) -> np.ndarray:
    out = np.zeros(len(lens) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    return out


def attend_rows(
    Q: np.ndarray,
    pos: np.ndarray,
    K: np.ndarray,
    V: np.ndarray,
    scale: float,
    causal: bool,
    key_lo: int = 0,
    key_hi: int | None = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """Attention of query rows against keys [key_lo, key_hi) of one KV head.

    Q: [r, D] float64 query rows; pos: [r] absolute position of each row in its
    context; K, V: [n, D] float64 keys and values of that context. Row t sees key j
    iff key_lo <= j < key_hi and, when causal, j <= pos[t].
    Returns O [r, D] float64 and LSE [r] float64 (natural log); a row that sees no
    key gets O = 0 and LSE = -inf.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.int64)
    r, d = Q.shape
    n = K.shape[0]
    hi = n if key_hi is None else min(int(key_hi), n)
    lo = max(0, int(key_lo))
    if causal:
        # No visible key lies beyond the furthest query position.
        hi = min(hi, int(pos.max()) + 1) if r else lo
    O = np.zeros((r, d), dtype=np.float64)
    LSE = np.full(r, -np.inf, dtype=np.float64)
    if r == 0 or hi <= lo:
        return O, LSE
    chunk = max(1, _CHUNK_ELEMS // max(1, r))

    def scores(j0: int, j1: int) -> np.ndarray:
        s = (Q @ K[j0:j1].T) * scale
        if causal:
            keys = np.arange(j0, j1, dtype=np.int64)
            s[keys[None, :] > pos[:, None]] = -np.inf
        return s

    # Pass 1: the global maximum score of each row.
    M = np.full(r, -np.inf, dtype=np.float64)
    for j0 in range(lo, hi, chunk):
        j1 = min(hi, j0 + chunk)
        M = np.maximum(M, scores(j0, j1).max(axis=1))
    seen = np.isfinite(M)
    Msafe = np.where(seen, M, 0.0)
    # Pass 2: sums of exp(s - M) and of exp(s - M) * v.
    den = np.zeros(r, dtype=np.float64)
    num = np.zeros((r, d), dtype=np.float64)
    for j0 in range(lo, hi, chunk):
        j1 = min(hi, j0 + chunk)
        p = np.exp(scores(j0, j1) - Msafe[:, None])
        den += p.sum(axis=1)
        num += p @ V[j0:j1]
    O[seen] = num[seen] / den[seen, None]
    LSE[seen] = M[seen] + np.log(den[seen])
    return O, LSE


def _group_rows(q_seq: np.ndarray, kappa: int, g: int) -> np.ndarray:
    """Query rows served by KV head kappa, ordered (query token, head in group)."""
    qs, _, d = q_seq.shape
    return q_seq[:, kappa * g:(kappa + 1) * g, :].reshape(qs * g, d)


def attention_ref(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    kv_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    causal: bool = True,
    scale: float | None = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """Unsharded attention of the whole batch.

    q: [sum q_s, Hq, D]; k, v: [sum n_s, Hkv, D] (float64, packed by sequence).
    Returns O [sum q_s, Hq, D] and LSE [sum q_s, Hq], float64.
    """
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = num_q_heads // num_kv_heads
    qo, ko = _offsets(q_lens), _offsets(kv_lens)
    O = np.zeros((q.shape[0], num_q_heads, d), dtype=np.float64)
    L = np.zeros((q.shape[0], num_q_heads), dtype=np.float64)
    for s, (n, qs) in enumerate(zip(kv_lens, q_lens)):
        pos = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)
        for kappa in range(num_kv_heads):
            rows = _group_rows(q[qo[s]:qo[s + 1]], kappa, g)
            o, lse = attend_rows(rows, pos, k[ko[s]:ko[s + 1], kappa], v[ko[s]:ko[s + 1], kappa], sc, causal)
            O[qo[s]:qo[s + 1], kappa * g:(kappa + 1) * g] = o.reshape(qs, g, d)
            L[qo[s]:qo[s + 1], kappa * g:(kappa + 1) * g] = lse.reshape(qs, g)
    return O, L


def partials_ref(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    kv_lens: Sequence[int],
    q_lens: Sequence[int],
    num_q_heads: int,
    num_kv_heads: int,
    block_len: int,
    causal: bool = True,
    scale: float | None = None,
) -> Dict[Tuple[int, int, int], Tuple[np.ndarray, np.ndarray]]:
    """Per-block partial results, keyed (sequence, block, KV head).

    Block b of sequence s holds keys [b*B, min((b+1)*B, n_s)) (fixed blocks from
    token 0; the last one may be short). Each value is (O_b [q_s, g, D], LSE_b
    [q_s, g]): attention restricted to that block's keys.
    """
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    g = num_q_heads // num_kv_heads
    qo, ko = _offsets(q_lens), _offsets(kv_lens)
    out: Dict[Tuple[int, int, int], Tuple[np.ndarray, np.ndarray]] = {}
    for s, (n, qs) in enumerate(zip(kv_lens, q_lens)):
        pos = np.repeat(np.arange(n - qs, n, dtype=np.int64), g)
        nb = -(-n // block_len)
        for kappa in range(num_kv_heads):
            rows = _group_rows(q[qo[s]:qo[s + 1]], kappa, g)
            ks, vs = k[ko[s]:ko[s + 1], kappa], v[ko[s]:ko[s + 1], kappa]
            for b in range(nb):
                o, lse = attend_rows(rows, pos, ks, vs, sc, causal, b * block_len, (b + 1) * block_len)
                out[(s, b, kappa)] = (o.reshape(qs, g, d), lse.reshape(qs, g))
    return out


def merge_ref(O_parts: np.ndarray, LSE_parts: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Log-sum-exp merge of partial results over the leading (block) axis.

    O_parts: [nb, ..., D]; LSE_parts: [nb, ...]. With M = max_b LSE_b and
    w_b = exp(LSE_b - M): O = sum_b w_b O_b / sum_b w_b and LSE = M + ln sum_b w_b.
    Since exp(LSE_b) O_b is block b's sum of exp(score) * value and exp(LSE_b) its
    sum of exp(score), this is exactly the unsharded softmax (the exactness the
    Split-KV page claims). Rows where every LSE_b is -inf get O = 0, LSE = -inf.
    """
    O_parts = np.asarray(O_parts, dtype=np.float64)
    LSE_parts = np.asarray(LSE_parts, dtype=np.float64)
    M = LSE_parts.max(axis=0)
    seen = np.isfinite(M)
    Msafe = np.where(seen, M, 0.0)
    w = np.exp(LSE_parts - Msafe[None])  # exp(-inf) = 0 for empty partials
    den = w.sum(axis=0)
    num = (w[..., None] * O_parts).sum(axis=0)
    O = np.zeros(O_parts.shape[1:], dtype=np.float64)
    LSE = np.full(LSE_parts.shape[1:], -np.inf, dtype=np.float64)
    O[seen] = num[seen] / den[seen][..., None]
    LSE[seen] = M[seen] + np.log(den[seen])
    return O, LSE


def sample_ref(
    q_seq: np.ndarray,
    k_seq: np.ndarray,
    v_seq: np.ndarray,
    pairs: List[Tuple[int, int]],
    num_kv_heads: int,
    causal: bool = True,
    scale: float | None = None,
) -> Tuple[np.ndarray, np.ndarray]:
    """Selected outputs of one sequence, for checks at sizes too large to run whole.

    q_seq: [q_s, Hq, D]; k_seq, v_seq: [n_s, Hkv, D]; pairs: (query index i, query
    head h). Returns O [len(pairs), D] and LSE [len(pairs)].
    """
    qs, hq, d = q_seq.shape
    n = k_seq.shape[0]
    g = hq // num_kv_heads
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    O = np.zeros((len(pairs), d), dtype=np.float64)
    L = np.zeros(len(pairs), dtype=np.float64)
    by_kv: Dict[int, List[int]] = {}
    for t, (i, h) in enumerate(pairs):
        by_kv.setdefault(h // g, []).append(t)
    for kappa, idx in by_kv.items():
        rows = np.stack([q_seq[pairs[t][0], pairs[t][1]] for t in idx])
        pos = np.array([n - qs + pairs[t][0] for t in idx], dtype=np.int64)
        o, lse = attend_rows(rows, pos, k_seq[:, kappa], v_seq[:, kappa], sc, causal)
        O[idx] = o
        L[idx] = lse
    return O, L
