"""GPU parity of the backward pass: libsplitkv's gradients against the float64 oracle.

The oracle evaluates the textbook gradients at the forward outputs the GPU produced
(O and LSE from splitkv_attn), so the comparison isolates the backward kernels. Small
cases run the whole oracle; a full-size workload is checked on sampled gradient rows.
"""

import time

import numpy as np
import pytest
import torch

import split_kv_exact_amd as skv
from oracle.backward import attention_grad_ref, grad_sample_ref
from tests.parity import compare_grads_whole, say
from workloads import Workload, get_workload, make_qkv, widen_to_f64

pytestmark = pytest.mark.gpu

# Tolerances (bf16 inputs; P and dS are rounded to bf16 before the matrix products, as
# P is in the forward): relative L2 error of each gradient tensor, and the largest
# element error relative to the tensor's largest magnitude. See the design notes for
# the derivation.
REL_L2 = 1e-2
REL_MAX = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _wl(name, kv, q, hq, hkv, d, b, m, causal=True, gran=0, seed=21, boost_frac=0.0):
    return Workload(name=name, dtype="bfloat16", kv_lens=tuple(kv), q_lens=tuple(q), num_q_heads=hq,
                    num_kv_heads=hkv, head_dim=d, block_len=b, num_workers=m, causal=causal, seed=seed,
                    boost_frac=boost_frac, boost=8.0, granularity=gran)


CASES = [
    _wl("ragged_d128", [1000, 333, 77, 2100, 16], [16, 5, 1, 40, 16], 32, 8, 128, 256, 16),
    _wl("ragged_d64", [1000, 333, 77, 513], [16, 5, 1, 9], 8, 2, 64, 128, 7),
    _wl("noncausal", [700, 45], [12, 3], 16, 4, 128, 128, 9, causal=False),
    _wl("whole_block_units", [900, 260], [8, 2], 16, 4, 128, 256, 6, gran=1),
    _wl("q_equals_n", [1, 5, 64, 2, 3], [1, 5, 64, 1, 3], 8, 4, 128, 16, 11),
    _wl("single_block", [100, 37], [3, 2], 8, 2, 128, 4096, 4),
    _wl("two_row_passes", [2048], [300], 32, 8, 128, 512, 8),
    _wl("boosted_keys", [3000, 1500], [16, 1], 64, 8, 128, 512, 32, boost_frac=0.01),
    _wl("mid_tiles", [700, 1200, 333], [5, 6, 7], 32, 2, 128, 256, 9),
    # Query heads per KV head that do not divide the 32-row chunk of the dK/dV kernel
    # (every chunk computes its rows' addresses): g = 3, and g = 64 (a chunk is half of
    # one query token's rows).
    _wl("group_of_3", [900, 300, 41], [7, 3, 2], 6, 2, 128, 256, 5),
    _wl("group_of_64", [500, 130], [3, 2], 64, 1, 64, 128, 4),
    # Many short sequences: 64-key tiles of 160 sequences found through the plan's tile
    # table, and dQ sums whose four-row groups straddle sequences.
    _wl("many_short_sequences", [(37 * i) % 400 + 1 for i in range(160)],
        [min((37 * i) % 400 + 1, 1 + i % 4) for i in range(160)], 6, 2, 128, 64, 32),
    # Sequences at the boundary of the few-row path (at most 16 query rows per KV head:
    # dK and dV from the dQ pass) and just past it, in one plan: g = 8 with q = 2 (16
    # rows) and q = 3 (24 rows); a one-key context; ragged 32-key stages; several blocks.
    _wl("few_row_boundary", [700, 45, 1, 33, 2049, 300], [2, 3, 1, 2, 2, 1], 16, 2, 128, 256, 9),
    # The few-row path at D = 64 without the causal mask, one- and multi-block.
    _wl("few_row_d64_noncausal", [300, 64, 513, 17], [1, 4, 2, 3], 8, 2, 64, 128, 5, causal=False),
]


def _do(wl, seed=99):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    return torch.randn((wl.total_q, wl.num_q_heads, wl.head_dim), generator=gen, device="cuda",
                       dtype=torch.float32).to(torch.bfloat16)


def _errors(got, ref):
    d = got - ref
    scale = max(np.abs(ref).max(), 1e-30)
    return float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)), float(np.abs(d).max() / scale)


def _forward_backward(wl, dkv_dtype=torch.float32):
    q, k, v = make_qkv(wl, "cuda")
    do = _do(wl)
    plan = skv.plan_for(wl)
    dev_plan = skv.splitkv_plan_upload(plan)
    out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v)
    ws = skv.workspace(plan)
    ws.fill_(float("nan"))
    dq = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    dk = torch.full(k.shape, float("nan"), dtype=dkv_dtype, device="cuda")
    dv = torch.full(v.shape, float("nan"), dtype=dkv_dtype, device="cuda")
    skv.splitkv_attn_backward(plan, dev_plan, q, k, v, do, out, lse, ws, dq, dk, dv)
    torch.cuda.synchronize()
    return q, k, v, do, out, lse, dq, dk, dv


# dK and dV stored as bf16: each is the fp32 result rounded to nearest even (tested
# bit for bit against the fp32 call), so the tolerance above still holds with a margin.
BF16_CASES = [CASES[0], CASES[4], CASES[7], CASES[9], CASES[11], CASES[12], CASES[13]]


@pytest.mark.parametrize("wl", BF16_CASES, ids=[w.name for w in BF16_CASES])
def test_bf16_dkv_is_the_rounded_fp32_result(wl):
    say(f"[gpu] backward {wl.name}, bf16 dK/dV")
    a = _forward_backward(wl)
    b = _forward_backward(wl, torch.bfloat16)
    assert torch.equal(a[6], b[6]), "dQ does not depend on the dK/dV dtype"
    for name, x, y in (("dk", a[7], b[7]), ("dv", a[8], b[8])):
        assert not torch.isnan(y).any(), f"{name} has unwritten entries"
        assert torch.equal(x.to(torch.bfloat16), y), name


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_small_backward_against_oracle(wl):
    say(f"[gpu] backward {wl.name}")
    q, k, v, do, out, lse, dq, dk, dv = _forward_backward(wl)
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(t).any(), f"{name} has unwritten entries"
    ref = attention_grad_ref(widen_to_f64(q), widen_to_f64(k), widen_to_f64(v), widen_to_f64(do), wl.kv_lens,
                             wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.causal,
                             o=widen_to_f64(out), lse=widen_to_f64(lse))
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        l2, mx = _errors(widen_to_f64(got), r)
        say(f"    {name}: rel L2 {l2:.2e}, max |d| / max |ref| {mx:.2e}")
        assert l2 <= REL_L2 and mx <= REL_MAX, (name, l2, mx)


def test_backward_is_deterministic():
    wl = CASES[0]
    a = _forward_backward(wl)
    b = _forward_backward(wl)
    for x, y in zip(a[6:], b[6:]):
        assert torch.equal(x, y)


def _full_seqs(wl, key):
    """Sequences whose gradients are sampled: the first and last, and for the mixed
    workloads decode and prefill ones; for the log-normal mix the shortest and longest
    contexts and the fewest and most queries."""
    if key == "mixed":
        return (0, 127, 128, 131)
    if key == "lognormal":
        return tuple(sorted({int(np.argmin(wl.kv_lens)), int(np.argmax(wl.kv_lens)), int(np.argmin(wl.q_lens)),
                             int(np.argmax(wl.q_lens))}))
    return tuple(sorted({0, wl.batch - 1}))


@pytest.mark.parametrize("key,dkv", [("batch8", "float32"), ("long", "float32"), ("lognormal", "float32"),
                                     ("decode", "float32"), ("mixed", "float32"), ("decode", "bfloat16"),
                                     ("mixed", "bfloat16")])
def test_full_size_backward_sampled(key, dkv):
    """Full-size workload in the benchmark's launch configuration, checked on sampled
    dQ rows and dK / dV keys of several sequences against the oracle at the GPU's
    forward outputs."""
    torch.cuda.empty_cache()
    wl = get_workload(key)
    say(f"[gpu] full-size backward {wl.name}, {dkv} dK/dV")
    q, k, v, do, out, lse, dq, dk, dv = _forward_backward(wl, getattr(torch, dkv))
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert not torch.isnan(t).any(), f"{name} has unwritten entries"
    rng = np.random.default_rng(5)
    qo = np.concatenate([[0], np.cumsum(wl.q_lens)])
    ko = np.concatenate([[0], np.cumsum(wl.kv_lens)])
    for s in _full_seqs(wl, key):
        n, qs = wl.kv_lens[s], wl.q_lens[s]
        pairs = sorted({(int(rng.integers(0, qs)), int(rng.integers(0, wl.num_q_heads))) for _ in range(6)}
                       | {(qs - 1, wl.num_q_heads - 1)})
        keys = sorted({(int(rng.integers(0, n)), int(rng.integers(0, wl.num_kv_heads))) for _ in range(6)}
                      | {(n - 1, 0), (0, wl.num_kv_heads - 1), (n - qs, wl.num_kv_heads // 2)})
        sl, kl = slice(qo[s], qo[s + 1]), slice(ko[s], ko[s + 1])
        rq, rk, rv = grad_sample_ref(widen_to_f64(q[sl]), widen_to_f64(k[kl]), widen_to_f64(v[kl]),
                                     widen_to_f64(do[sl]), widen_to_f64(out[sl]), widen_to_f64(lse[sl]),
                                     wl.num_kv_heads, pairs, keys, wl.causal)
        gq = np.stack([widen_to_f64(dq[qo[s] + i, h]) for i, h in pairs])
        gk = np.stack([widen_to_f64(dk[ko[s] + j, c]) for j, c in keys])
        gv = np.stack([widen_to_f64(dv[ko[s] + j, c]) for j, c in keys])
        for name, got, r in (("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)):
            l2, mx = _errors(got, r)
            say(f"    seq {s} {name}: rel L2 {l2:.2e}, max |d| / max |ref| {mx:.2e}")
            assert l2 <= REL_L2 and mx <= REL_MAX, (s, name, l2, mx)
    del q, k, v, do, out, lse, dq, dk, dv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key,dkv,part", [("batch8", "float32", "all"), ("long", "float32", "all"),
                                          ("lognormal", "float32", "all"), ("decode", "bfloat16", "all"),
                                          ("mixed", "float32", "decode"), ("mixed", "bfloat16", "prefill")])
def test_full_size_backward_whole(key, dkv, part):
    """Full-size workload in the benchmark's launch configuration, every gradient entry
    against the float64 oracle at the GPU's forward outputs (the mixed batch in two
    parts: its 128 decode sequences, then its 4 prefill chunks): relative L2 over each
    whole tensor and the largest element error against its largest magnitude."""
    torch.cuda.empty_cache()
    wl = get_workload(key)
    seqs = {"all": None, "decode": range(128), "prefill": range(128, 132)}[part]
    say(f"[gpu] full-size backward {wl.name}, {dkv} dK/dV, whole tensors ({part})")
    q, k, v, do, out, lse, dq, dk, dv = _forward_backward(wl, getattr(torch, dkv))
    t0 = time.time()
    res = compare_grads_whole(wl, q, k, v, do, out, lse, dq, dk, dv, seqs=seqs)
    say(f"    {time.time() - t0:.0f} s: {res}")
    for name in ("dq", "dk", "dv"):
        l2, mx = res.errors(name)
        assert l2 <= REL_L2 and mx <= REL_MAX, (name, l2, mx)
    del q, k, v, do, out, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_caller_scale_forward_and_backward():
    """A softmax scale other than 1/sqrt(D) (0.3 here, 3.4 times the default for D = 128,
    so the softmax is much sharper) passed to the forward and the backward call, against
    the oracle with the same scale; the case has jobs of every forward and backward path."""
    from oracle import attention_ref
    from tests.parity import assert_within, compare

    wl, sc = CASES[0], 0.3
    say(f"[gpu] forward and backward with scale {sc}, {wl.name}")
    q, k, v = make_qkv(wl, "cuda")
    do = _do(wl)
    plan = skv.plan_for(wl)
    dev_plan = skv.splitkv_plan_upload(plan)
    out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v, scale=sc)
    dq, dk, dv = skv.splitkv_attn_backward(plan, dev_plan, q, k, v, do, out, lse, scale=sc)
    torch.cuda.synchronize()
    O, L = attention_ref(widen_to_f64(q), widen_to_f64(k), widen_to_f64(v), wl.kv_lens, wl.q_lens,
                         wl.num_q_heads, wl.num_kv_heads, wl.causal, scale=sc)
    d = compare(out.cpu().numpy(), O, lse.cpu().numpy(), L)
    say(f"    forward: {d}")
    assert_within(d, wl.dtype, "forward with a caller scale")
    ref = attention_grad_ref(widen_to_f64(q), widen_to_f64(k), widen_to_f64(v), widen_to_f64(do), wl.kv_lens,
                             wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.causal, scale=sc,
                             o=widen_to_f64(out), lse=widen_to_f64(lse))
    for name, got, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        l2, mx = _errors(widen_to_f64(got), r)
        say(f"    {name}: rel L2 {l2:.2e}, max |d| / max |ref| {mx:.2e}")
        assert l2 <= REL_L2 and mx <= REL_MAX, (name, l2, mx)
