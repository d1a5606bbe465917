"""The five workload shapes of the exact split-KV problem, as seeded data.

Each workload is a batch of sequences. Sequence s has a context of n_s key/value
tokens and q_s query tokens; the queries are the last q_s tokens of that context.
Lengths are drawn with numpy's PCG64 generator from a fixed seed, so a workload is
reproducible from its name alone.

The shapes follow the problem the Split-KV page sets out in its lede: very short
query blocks over very long contexts, with the context cut into KV blocks that are
placed on workers by a cost-aware LPT plan. Where the shapes leave a choice open
(inclusive bounds, rounding, worker counts, the block size of the mixed batch, which
keys are boosted) the reading taken is stated next to the generator.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, Tuple

import numpy as np

# Plan granularities, matching the library's enum values.
UNIT_SEQ_BLOCK_KVHEAD = 0
UNIT_SEQ_BLOCK = 1


@dataclass(frozen=True)
class Workload:
    """One split-KV problem instance (shapes and seeds; tensors come from ``make_qkv``)."""

    name: str
    dtype: str  # "float32" or "bfloat16"
    kv_lens: Tuple[int, ...]
    q_lens: Tuple[int, ...]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_len: int
    num_workers: int
    causal: bool = True
    seed: int = 0
    # Fraction of (token, kv-head) key rows multiplied by ``boost`` before the cast.
    boost_frac: float = 0.0
    boost: float = 1.0
    granularity: int = UNIT_SEQ_BLOCK_KVHEAD
    note: str = field(default="", compare=False)

    @property
    def batch(self) -> int:
        return len(self.kv_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def total_kv(self) -> int:
        return int(sum(self.kv_lens))

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "float32" else 2

    def num_blocks(self, s: int) -> int:
        return -(-self.kv_lens[s] // self.block_len)

    def with_workers(self, m: int) -> "Workload":
        return _replace(self, num_workers=m)

    def with_block(self, b: int) -> "Workload":
        return _replace(self, block_len=b)

    def summary(self) -> dict:
        return {
            "workload": self.name,
            "dtype": self.dtype,
            "batch": self.batch,
            "sum_kv_tokens": self.total_kv,
            "sum_q_tokens": self.total_q,
            "q_heads": self.num_q_heads,
            "kv_heads": self.num_kv_heads,
            "head_dim": self.head_dim,
            "block_len": self.block_len,
            "workers": self.num_workers,
            "causal": self.causal,
            "seed": self.seed,
        }


def _replace(wl: Workload, **kw) -> Workload:
    from dataclasses import replace

    return replace(wl, **kw)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# The five workloads. Integer uniform draws use inclusive bounds.
# ---------------------------------------------------------------------------


def small_fp32(seed: int = 1001) -> Workload:
    """fp32, one sequence, 1 query head / 1 KV head, head_dim 64: 4 trailing causal
    queries over a 2048-token context cut into 8 blocks of 256. Reading: 8 workers,
    one block each, since the shape names 8 blocks and 8 partials and no worker count."""
    return Workload(
        name="small_fp32_1x2048_q4_d64",
        dtype="float32",
        kv_lens=(2048,),
        q_lens=(4,),
        num_q_heads=1,
        num_kv_heads=1,
        head_dim=64,
        block_len=256,
        num_workers=8,
        seed=seed,
    )


def batch8_bf16(seed: int = 1002) -> Workload:
    """bf16, 8 sequences with contexts uniform in [4096, 32768], 16 trailing causal
    queries, GQA 32/8, head_dim 128, KV block 512, LPT over 256 workers."""
    r = _rng(seed)
    n = r.integers(4096, 32768, size=8, endpoint=True)
    return Workload(
        name="batch8_bf16_ctx4k-32k_q16_gqa32-8_d128_b512",
        dtype="bfloat16",
        kv_lens=tuple(int(x) for x in n),
        q_lens=(16,) * 8,
        num_q_heads=32,
        num_kv_heads=8,
        head_dim=128,
        block_len=512,
        num_workers=256,
        seed=seed,
    )


def long_context_bf16(seed: int = 1003) -> Workload:
    """bf16, one sequence of 1,048,576 context tokens, 64 trailing causal queries,
    GQA 64/8, head_dim 128, KV block 4096 (4 GiB of K+V)."""
    return Workload(
        name="long_bf16_ctx1M_q64_gqa64-8_d128_b4096",
        dtype="bfloat16",
        kv_lens=(1 << 20,),
        q_lens=(64,),
        num_q_heads=64,
        num_kv_heads=8,
        head_dim=128,
        block_len=4096,
        num_workers=256,
        seed=seed,
    )


def lognormal_mix_bf16(seed: int = 1004) -> Workload:
    """bf16, 64 sequences; context lengths log-normal with median 16384 and sigma 1.0,
    rounded to the nearest integer and clipped to [1024, 262144]; query counts uniform
    in [1, 128]; GQA 32/8, head_dim 128, KV block 1024, LPT over 256 workers."""
    r = _rng(seed)
    z = r.standard_normal(64)
    n = np.clip(np.rint(np.exp(math.log(16384.0) + 1.0 * z)), 1024, 262144).astype(np.int64)
    q = r.integers(1, 128, size=64, endpoint=True)
    return Workload(
        name="lognormal64_bf16_med16k_q1-128_gqa32-8_d128_b1024",
        dtype="bfloat16",
        kv_lens=tuple(int(x) for x in n),
        q_lens=tuple(int(x) for x in q),
        num_q_heads=32,
        num_kv_heads=8,
        head_dim=128,
        block_len=1024,
        num_workers=256,
        seed=seed,
    )


def _mixed_decode_lens(seed: int) -> np.ndarray:
    r = _rng(seed)
    return r.integers(8192, 131072, size=128, endpoint=True)


def mixed_decode_prefill_bf16(seed: int = 1005) -> Workload:
    """bf16 mixed batch: 128 decode sequences (1 query, context uniform in [8192,
    131072]) followed by 4 prefill chunks (the last 2048 tokens of 65536-token
    contexts, causal on the chunk). GQA 64/8, head_dim 128. Readings: KV block 8192
    (the shape gives none: the largest block that still gives every worker a prefill
    unit, so the fewest partials for the exact merge); 0.1% of (token, kv-head) key
    rows, drawn Bernoulli, are multiplied by 8 before the bf16 cast (a power of two, so
    the cast stays exact)."""
    n_dec = _mixed_decode_lens(seed)
    kv = tuple(int(x) for x in n_dec) + (65536,) * 4
    q = (1,) * 128 + (2048,) * 4
    return Workload(
        name="mixed_bf16_128dec-ctx8k-128k_4prefill-2048of64k_gqa64-8_d128_b8192",
        dtype="bfloat16",
        kv_lens=kv,
        q_lens=q,
        num_q_heads=64,
        num_kv_heads=8,
        head_dim=128,
        block_len=8192,
        num_workers=256,
        seed=seed,
        boost_frac=0.001,
        boost=8.0,
    )


def decode_only_bf16(seed: int = 1005) -> Workload:
    """The 128 decode sequences of the mixed batch on their own: same seed, same
    context lengths, KV block and tensor recipe (boosted keys included), without the
    prefill chunks. This is the memory-bound part of that batch."""
    n_dec = _mixed_decode_lens(seed)
    return Workload(
        name="decode128_bf16_ctx8k-128k_q1_gqa64-8_d128_b8192",
        dtype="bfloat16",
        kv_lens=tuple(int(x) for x in n_dec),
        q_lens=(1,) * 128,
        num_q_heads=64,
        num_kv_heads=8,
        head_dim=128,
        block_len=8192,
        num_workers=256,
        seed=seed,
        boost_frac=0.001,
        boost=8.0,
    )


WORKLOADS: Dict[str, Callable[[], Workload]] = {
    "small": small_fp32,
    "batch8": batch8_bf16,
    "long": long_context_bf16,
    "lognormal": lognormal_mix_bf16,
    "mixed": mixed_decode_prefill_bf16,
    "decode": decode_only_bf16,
}


def get_workload(key: str) -> Workload:
    try:
        return WORKLOADS[key]()
    except KeyError:
        raise KeyError(f"unknown workload {key!r}; choose from {sorted(WORKLOADS)}") from None
