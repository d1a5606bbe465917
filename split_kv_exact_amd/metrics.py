"""Byte and flop accounting for throughput reports (counting only).

effective_bytes: what the whole split-KV attention must move at least once:
    Q + K + V (each stored element counted once) + O (fp32) + LSE (fp32).
partial_kernel_bytes: what one launch of the partial-attention kernel must move:
    per unit (sequence s, block b, KV heads), the block's K and V, the unit's query
    rows of Q, and its partial output and LSE in the plan's partial format.
merge_kernel_bytes: partials read once, O and LSE written once.
partial_traffic_bytes: the partial outputs and LSEs written by the partial kernel and
    read back by the merge, 2 * partial_rows * row bytes: (D + 1) * 4 for fp32 partials
    (fp32 inputs), D * 2 + 8 for row-scaled fp16 partials (bf16 inputs: fp16 elements,
    the LSE and the row scale). This is traffic the exact merge costs, never credited
    as useful bytes.
flops: 2 flops per multiply-add of QK^T and of PV over the (query, key) pairs the
    mask keeps: 4 * D * Hq * sum_s visible_pairs_s.
"""

from __future__ import annotations

# MI355X published peaks used for roofline fractions.
PEAK_HBM_GBS = 8000.0
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_FP32_VECTOR_TFLOPS = 157.3


def visible_pairs(wl) -> int:
    tot = 0
    for n, q in zip(wl.kv_lens, wl.q_lens):
        tot += q * n - q * (q - 1) // 2 if wl.causal else q * n
    return tot


def flops(wl) -> int:
    return 4 * wl.head_dim * wl.num_q_heads * visible_pairs(wl)


def kv_bytes(wl) -> int:
    return 2 * wl.total_kv * wl.num_kv_heads * wl.head_dim * wl.elem_bytes


def q_bytes(wl) -> int:
    return wl.total_q * wl.num_q_heads * wl.head_dim * wl.elem_bytes


def out_bytes(wl) -> int:
    return wl.total_q * wl.num_q_heads * (wl.head_dim + 1) * 4


def effective_bytes(wl) -> int:
    return q_bytes(wl) + kv_bytes(wl) + out_bytes(wl)


def partial_rows(wl) -> int:
    return sum(wl.num_blocks(s) * wl.num_kv_heads * wl.q_lens[s] * wl.group for s in range(wl.batch))


def partial_kernel_bytes(wl) -> int:
    q_per_unit = sum(wl.num_blocks(s) * wl.q_lens[s] * wl.num_q_heads for s in range(wl.batch))
    return kv_bytes(wl) + q_per_unit * wl.head_dim * wl.elem_bytes + partial_rows(wl) * partial_row_bytes(wl)


def partial_row_bytes(wl) -> int:
    """Bytes of one stored partial row in the format the plans of this workload use."""
    return wl.head_dim * 2 + 8 if wl.dtype == "bfloat16" else (wl.head_dim + 1) * 4


def partial_traffic_bytes(wl) -> int:
    return 2 * partial_rows(wl) * partial_row_bytes(wl)


def merge_kernel_bytes(wl) -> int:
    return partial_rows(wl) * partial_row_bytes(wl) + out_bytes(wl)


def roofline_seconds(wl) -> float:
    peak_f = PEAK_FP32_VECTOR_TFLOPS if wl.dtype == "float32" else PEAK_BF16_MFMA_TFLOPS
    return max(effective_bytes(wl) / (PEAK_HBM_GBS * 1e9), flops(wl) / (peak_f * 1e12))


def peak_flops_tflops(wl) -> float:
    return PEAK_FP32_VECTOR_TFLOPS if wl.dtype == "float32" else PEAK_BF16_MFMA_TFLOPS


def binding_roof(wl) -> str:
    peak_f = PEAK_FP32_VECTOR_TFLOPS if wl.dtype == "float32" else PEAK_BF16_MFMA_TFLOPS
    return "hbm" if effective_bytes(wl) / (PEAK_HBM_GBS * 1e9) >= flops(wl) / (peak_f * 1e12) else "mfma"


def backward_flops(wl) -> int:
    """Backward pass: five products per visible (row, key) pair and dimension pair of
    multiply-adds (S = Q K^T recomputed, dP = dO V^T, dV = P^T dO, dK = dS^T Q,
    dQ = dS K), 10 * D flops per pair: 2.5 times the forward."""
    return 10 * wl.head_dim * wl.num_q_heads * visible_pairs(wl)


def backward_bytes(wl, dkv_bytes: int = 4) -> int:
    """Backward pass, each element once: Q, K, V and dO read in the input dtype, O and
    LSE read and dQ written in fp32, dK and dV written with ``dkv_bytes`` per element
    (4 for fp32, 2 for bf16)."""
    es = 2 if wl.dtype == "bfloat16" else 4
    d = wl.head_dim
    q_elems = wl.total_q * wl.num_q_heads * d
    kv_elems = wl.total_kv * wl.num_kv_heads * d
    return (2 * q_elems + 2 * kv_elems) * es + (q_elems + wl.total_q * wl.num_q_heads) * 4 \
        + q_elems * 4 + 2 * kv_elems * dkv_bytes


def backward_roofline_seconds(wl, dkv_bytes: int = 4) -> float:
    return max(backward_bytes(wl, dkv_bytes) / (PEAK_HBM_GBS * 1e9),
               backward_flops(wl) / (PEAK_BF16_MFMA_TFLOPS * 1e12))
