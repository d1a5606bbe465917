"""GPU parity: libsplitkv's HIP kernels against the float64 oracle (needs an MI355X).

Small cases run the whole oracle (every output, every partial). The five workload
shapes and the decode-only batch at full size are compared whole (every output row),
with sampled partials, in the launch configuration the benchmark times (the fused
call over the LPT plan). Inputs are drawn on the device and copied to the host for
the oracle.
"""

import math

import numpy as np
import pytest
import torch

import split_kv_exact_amd as skv
from oracle import attend_rows, attention_ref, partials_ref
from tests.parity import Diff, assert_fused_matches_merge, assert_within, compare, compare_whole, offsets, partial_row, say, scale_of
from workloads import Workload, get_workload, make_qkv, widen_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _wl(name, kv, q, hq, hkv, d, b, m, dtype="bfloat16", causal=True, gran=0, seed=7, boost_frac=0.0):
    return Workload(name=name, dtype=dtype, kv_lens=tuple(kv), q_lens=tuple(q), num_q_heads=hq, num_kv_heads=hkv,
                    head_dim=d, block_len=b, num_workers=m, causal=causal, seed=seed, boost_frac=boost_frac,
                    boost=8.0, granularity=gran)


MANY_KV = [(37 * i) % 400 + 1 for i in range(240)]
MANY_Q = [min(n, 1 + i % 4) for i, n in enumerate(MANY_KV)]

SMALL = [
    get_workload("small"),
    _wl("ragged_bf16_d128", [1000, 333, 77, 2100, 16], [16, 5, 1, 40, 16], 32, 8, 128, 256, 16),
    _wl("ragged_bf16_d64", [1000, 333, 77, 513], [16, 5, 1, 9], 8, 2, 64, 128, 7),
    _wl("fp32_d128", [300, 129, 64], [7, 3, 64], 4, 2, 128, 64, 5, dtype="float32"),
    _wl("noncausal_bf16", [700, 45], [12, 3], 16, 4, 128, 128, 9, causal=False),
    _wl("noncausal_fp32_d64", [200, 45], [4, 3], 2, 1, 64, 64, 3, dtype="float32", causal=False),
    _wl("whole_block_units", [900, 260], [8, 2], 16, 4, 128, 256, 6, gran=1),
    _wl("edge_q_equals_n", [1, 5, 64, 2, 3], [1, 5, 64, 1, 3], 8, 4, 128, 16, 11),
    _wl("block_longer_than_context", [100, 37], [3, 2], 8, 2, 128, 4096, 4),
    _wl("boosted_keys", [3000, 1500], [16, 1], 64, 8, 128, 512, 32, boost_frac=0.01),
    _wl("many_rows", [2048], [300], 32, 8, 128, 512, 8),
    _wl("more_workers_than_units", [300], [2], 4, 1, 128, 128, 64),
    # Multi-job units dealt over the workers of an XCD class (needs >= 16 workers).
    _wl("multi_pass_dealt", [2048, 900, 5000], [300, 70, 16], 32, 8, 128, 512, 32),
    _wl("whole_block_dealt", [900, 260, 3000], [8, 2, 33], 16, 4, 128, 256, 16, gran=1),
    # 5, 6 and 7 row tiles per job (GQA group 16): waves 0-3 hold one or two tiles each.
    _wl("mid_tiles_d128", [700, 1200, 333], [5, 6, 7], 32, 2, 128, 256, 9),
    _wl("mid_tiles_d64", [700, 1200, 333], [5, 6, 7], 32, 2, 64, 128, 9),
    # Matrix-path jobs whose passes all have 16 row tiles (the kernel variant without
    # per-wave tile skipping): 256-row units, 500- and 504-row units (two passes, ragged
    # last tile), small jobs beside them; D 128 and 64, causal and not, q = n, boosted
    # keys.
    _wl("full_passes_d128", [3000, 700, 1500], [64, 125, 20], 32, 8, 128, 512, 16),
    _wl("full_passes_d64", [1100, 2000, 90], [32, 63, 3], 16, 2, 64, 256, 9, causal=False),
    _wl("full_passes_q_equals_n", [64, 300], [64, 64], 16, 4, 128, 128, 8),
    _wl("full_passes_boosted", [5000], [64], 64, 8, 128, 1024, 16, boost_frac=0.01),
    # A GQA group that is not a power of two (g = 3) and one of 64 heads per KV head.
    _wl("group_of_3", [900, 300, 41], [7, 3, 2], 6, 2, 128, 256, 5),
    _wl("group_of_64", [500, 130], [3, 2], 64, 1, 64, 128, 4),
    # Many short sequences, one to seven 64-key blocks, 6 to 24 rows per sequence: merge
    # workgroups (four rows) often straddle two sequences, in both the merge of every
    # sequence and the fused call's merge of the multi-block ones.
    _wl("many_short_sequences", MANY_KV, MANY_Q, 6, 2, 128, 64, 32),
]
# Matrix-path kernel variant each case must run (mma_partial_passes of the plan info).
MMA_PARTIAL_PASSES = {"full_passes_d128": 0, "full_passes_d64": 0, "full_passes_q_equals_n": 0,
                      "full_passes_boosted": 0, "many_rows": 1, "multi_pass_dealt": 1, "boosted_keys": 1}


def _run_all(wl, q, k, v, m=None):
    plan = skv.plan_for(wl if m is None else wl.with_workers(m))
    dev_plan = skv.splitkv_plan_upload(plan)
    ws = skv.workspace(plan)
    ws.fill_(float("nan"))
    skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws)
    out_m = torch.full((wl.total_q, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
    lse_m = torch.full((wl.total_q, wl.num_q_heads), float("nan"), device="cuda")
    skv.splitkv_merge(plan, dev_plan, ws, out_m, lse_m)
    ws2 = skv.workspace(plan)
    ws2.fill_(float("nan"))
    out_f = torch.full_like(out_m, float("nan"))
    lse_f = torch.full_like(lse_m, float("nan"))
    skv.splitkv_attn(plan, dev_plan, q, k, v, ws2, out_f, lse_f)
    torch.cuda.synchronize()
    return plan, ws, out_m, lse_m, out_f, lse_f


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_cases_against_full_oracle(wl):
    say(f"[gpu] small case {wl.name}")
    q, k, v = make_qkv(wl, "cuda")
    plan, ws, out_m, lse_m, out_f, lse_f = _run_all(wl, q, k, v)
    if wl.name in MMA_PARTIAL_PASSES:
        inf = plan.info()
        assert inf["num_mma_jobs"] > 0 and inf["mma_partial_passes"] == MMA_PARTIAL_PASSES[wl.name]
    qh, kh, vh = widen_to_f64(q), widen_to_f64(k), widen_to_f64(v)
    O, L = attention_ref(qh, kh, vh, wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.causal)
    d_merge = compare(out_m.cpu().numpy(), O, lse_m.cpu().numpy(), L)
    d_fused = compare(out_f.cpu().numpy(), O, lse_f.cpu().numpy(), L)
    say(f"  merge: {d_merge}\n  fused: {d_fused}")
    assert_within(d_merge, wl.dtype, "partial+merge")
    assert_within(d_fused, wl.dtype, "fused")
    # The fused call writes single-block sequences directly; all other rows go through
    # the same merge.
    assert_fused_matches_merge(wl, plan, out_f, lse_f, out_m, lse_m)
    # Every partial against the oracle's per-block partials.
    parts = partials_ref(qh, kh, vh, wl.kv_lens, wl.q_lens, wl.num_q_heads, wl.num_kv_heads, wl.block_len,
                         wl.causal)
    wo, wlse = skv.workspace_views(plan, ws)
    wo, wlse = wo.cpu().numpy(), wlse.cpu().numpy()
    assert not np.any(np.isnan(wlse)), "workspace LSE left unwritten"
    g = wl.group
    go, gl, ro, rl = [], [], [], []
    for (s, b, kap), (Ob, Lb) in parts.items():
        r0 = partial_row(wl, s, b, kap, 0)
        rows = wl.q_lens[s] * g
        go.append(wo[r0:r0 + rows])
        gl.append(wlse[r0:r0 + rows])
        ro.append(Ob.reshape(rows, wl.head_dim))
        rl.append(Lb.reshape(rows))
    d_part = compare(np.concatenate(go), np.concatenate(ro), np.concatenate(gl), np.concatenate(rl))
    say(f"  partials: {d_part}")
    assert_within(d_part, wl.dtype, "partials")


def test_bitwise_identical_across_worker_counts():
    wl = SMALL[1]
    say(f"[gpu] worker-count invariance on {wl.name}")
    q, k, v = make_qkv(wl, "cuda")
    ref = None
    for m in (1, 3, 16, 256):
        _, _, out_m, lse_m, out_f, lse_f = _run_all(wl, q, k, v, m)
        if ref is None:
            ref = (out_f.clone(), lse_f.clone(), out_m.clone(), lse_m.clone())
        assert torch.equal(out_f, ref[0]) and torch.equal(lse_f, ref[1]), f"m={m}"
        assert torch.equal(out_m, ref[2]) and torch.equal(lse_m, ref[3]), f"m={m}"


@pytest.mark.parametrize("name", ["ragged_bf16_d128", "ragged_bf16_d64", "many_rows", "edge_q_equals_n",
                                  "many_short_sequences"])
def test_bf16_partial_formats_agree(name):
    """bf16 inputs under both partial formats: fp32 partials meet the oracle, the LSEs of
    the two formats are the same bits, and each fp16 element, decoded with its row scale,
    lies within half an fp16 step at 1.0 (2^-12) of the row's largest |O| from the fp32
    partial."""
    wl = next(w for w in SMALL if w.name == name)
    say(f"[gpu] partial formats on {wl.name}")
    q, k, v = make_qkv(wl, "cuda")
    got = {}
    for fmt in (skv.SPLITKV_PARTIAL_F32, skv.SPLITKV_PARTIAL_F16_ROWSCALE):
        plan = skv.plan_for(wl, partial_format=fmt)
        assert plan.info()["partial_format"] == fmt
        dev_plan = skv.splitkv_plan_upload(plan)
        ws = skv.workspace(plan)
        ws.fill_(float("nan"))
        skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws)
        out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v)
        torch.cuda.synchronize()
        wo, wlse = skv.workspace_views(plan, ws)
        got[fmt] = (wo.cpu().numpy(), wlse.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy())
    f32, h16 = got[skv.SPLITKV_PARTIAL_F32], got[skv.SPLITKV_PARTIAL_F16_ROWSCALE]
    O, L = attention_ref(widen_to_f64(q), widen_to_f64(k), widen_to_f64(v), wl.kv_lens, wl.q_lens,
                         wl.num_q_heads, wl.num_kv_heads, wl.causal)
    d = compare(f32[2], O, f32[3], L)
    say(f"  fp32 partials, fused: {d}")
    assert_within(d, wl.dtype, "fused with fp32 partials")
    assert not np.any(np.isnan(f32[1])) and np.array_equal(f32[1], h16[1])
    rowmax = np.abs(f32[0]).max(axis=1, keepdims=True)
    err = np.abs(h16[0] - f32[0])
    assert np.all(err <= rowmax * (2.0 ** -12 * 1.001) + 1e-30), float((err / np.maximum(rowmax, 1e-30)).max())
    assert np.array_equal(f32[3], h16[3])  # the merged LSE depends on the partial LSEs only


def test_repeated_calls_reuse_buffers():
    wl = SMALL[2]
    say(f"[gpu] repeated calls on {wl.name}")
    q, k, v = make_qkv(wl, "cuda")
    plan = skv.plan_for(wl)
    dev_plan = skv.splitkv_plan_upload(plan)
    ws = skv.workspace(plan)
    outs = [skv.splitkv_attn(plan, dev_plan, q, k, v, ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


def _schedules_agree(wl, q, k, v, m=None):
    """Partials and fused outputs under every job schedule, under a plan built with the
    roofline-aware cost (other placement, same jobs), and under one whose workers are
    re-placed by XCD speeds, bit for bit; afterwards the plan buffers' scheduling areas
    (their last 1024 bytes) are zero again."""
    w = wl if m is None else wl.with_workers(m)
    res = {}
    speeds = [1000, 900, 1000, 970, 1000, 910, 990, 1000]
    for ridge, sp, scheds in ((0, None, ("static", "queue", "queue", "auto")), (128, None, ("static", "queue")),
                              (0, speeds, ("static", "queue"))):
        plan = skv.plan_for(w, ridge, sp)
        dev_plan = skv.splitkv_plan_upload(plan)
        for sched in scheds:
            ws = skv.workspace(plan)
            ws.fill_(float("nan"))
            skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws, schedule=sched)
            out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v, schedule=sched)
            wo, wlse = skv.workspace_views(plan, ws)
            res.setdefault((ridge, sp is not None, sched), []).append((wo, wlse, out, lse))
        torch.cuda.synchronize()
        assert int(dev_plan[-1024:].count_nonzero()) == 0, "scheduling area not left zero"
    ref = res[(0, False, "static")][0]
    assert not torch.isnan(ref[1]).any()
    for key, runs in res.items():
        for got in runs:
            for a, b in zip(got, ref):
                assert torch.equal(a, b), key


@pytest.mark.parametrize("wl", [w for w in SMALL if w.dtype == "bfloat16"],
                         ids=[w.name for w in SMALL if w.dtype == "bfloat16"])
def test_static_and_queue_schedules_agree(wl):
    say(f"[gpu] schedules on {wl.name}")
    q, k, v = make_qkv(wl, "cuda")
    _schedules_agree(wl, q, k, v)


def test_xcd_placement_fp32_agrees():
    """The float32 kernel walks each workgroup's units; re-placed workers give the same
    partials bit for bit."""
    for wl in [w for w in SMALL if w.dtype == "float32"]:
        say(f"[gpu] XCD placement on {wl.name}")
        q, k, v = make_qkv(wl, "cuda")
        got = []
        for sp in (None, [1000, 1, 500, 999, 1000, 2, 800, 1000]):
            plan = skv.plan_for(wl, 0, sp)
            dev_plan = skv.splitkv_plan_upload(plan)
            ws = skv.workspace(plan)
            ws.fill_(float("nan"))
            skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws)
            out, lse = skv.splitkv_attn(plan, dev_plan, q, k, v)
            got.append((*skv.workspace_views(plan, ws), out, lse))
        torch.cuda.synchronize()
        for a, b in zip(*got):
            assert torch.equal(a, b)


def test_worker_clock():
    for wl in (SMALL[1], SMALL[0]):  # bf16 and fp32 kernels
        say(f"[gpu] worker clock on {wl.name}")
        q, k, v = make_qkv(wl, "cuda")
        plan = skv.plan_for(wl)
        dev_plan = skv.splitkv_plan_upload(plan)
        clock = torch.zeros(2 * wl.num_workers, dtype=torch.int64, device="cuda")
        skv.splitkv_partial_attn(plan, dev_plan, q, k, v, clock=clock)
        torch.cuda.synchronize()
        c = clock.view(-1, 2).cpu()
        assert bool((c[:, 0] > 0).all()) and bool((c[:, 1] >= c[:, 0]).all())


# --------------------------------------------------------------------------- full sizes
#
# Every workload at full size through the fused call over its LPT plan (the launch the
# benchmark times). Outputs are compared with the float64 oracle over the whole output
# (streamed per sequence, several host threads); partials are compared on sampled rows
# of sampled blocks.

_FULL = {}


def _full(key):
    """Inputs, plan and fused outputs of one full-size workload (cached while the next
    test uses the same workload); the separate calls must give the same bits."""
    if key in _FULL:
        return _FULL[key]
    _FULL.clear()
    torch.cuda.empty_cache()
    wl = get_workload(key)
    say(f"[gpu] full-size {wl.name}: drawing inputs")
    q, k, v = make_qkv(wl, "cuda")
    plan = skv.plan_for(wl)
    dev_plan = skv.splitkv_plan_upload(plan)
    ws = skv.workspace(plan)
    out = torch.full((wl.total_q, wl.num_q_heads, wl.head_dim), float("nan"), device="cuda")
    lse = torch.full((wl.total_q, wl.num_q_heads), float("nan"), device="cuda")
    say(f"[gpu] full-size {wl.name}: fused call")
    skv.splitkv_attn(plan, dev_plan, q, k, v, ws, out, lse)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any() and torch.isfinite(lse).all(), "unwritten or non-finite outputs"
    say(f"[gpu] full-size {wl.name}: separate calls")
    ws.fill_(float("nan"))
    skv.splitkv_partial_attn(plan, dev_plan, q, k, v, ws)
    out2, lse2 = skv.splitkv_merge(plan, dev_plan, ws)
    torch.cuda.synchronize()
    assert_fused_matches_merge(wl, plan, out, lse, out2, lse2)
    del out2, lse2
    _FULL[key] = (wl, q, k, v, plan, ws, out, lse)
    return _FULL[key]


def _whole(key, seqs=None, what=""):
    wl, q, k, v, plan, ws, out, lse = _full(key)
    say(f"[gpu] full-size {wl.name}{what}: whole output against the oracle")
    d = compare_whole(wl, q, k, v, out, lse, seqs=seqs, rows_per_task=1024)
    say(f"  whole output{what} ({wl.total_q if seqs is None else sum(wl.q_lens[s] for s in seqs)} query tokens "
        f"x {wl.num_q_heads} heads): {d}")
    assert_within(d, wl.dtype, f"{wl.name}{what} whole output")
    return d


def _sample_pairs(rng, wl, s, count):
    qs = wl.q_lens[s]
    pairs = {(qs - 1, int(rng.integers(0, wl.num_q_heads))), (0, int(rng.integers(0, wl.num_q_heads)))}
    while len(pairs) < min(count, qs * wl.num_q_heads):
        pairs.add((int(rng.integers(0, qs)), int(rng.integers(0, wl.num_q_heads))))
    return sorted(pairs)


def _check_partials_sampled(key, seqs, per_seq, seed=0):
    """Partials of sampled rows (first, last and one middle block of each sampled
    sequence) against the oracle's per-block attention, read at their ABI rows."""
    wl, q, k, v, plan, ws, out, lse = _full(key)
    wo, wlse = skv.workspace_views(plan, ws)
    rng = np.random.default_rng(seed)
    qo, ko = offsets(wl.q_lens), offsets(wl.kv_lens)
    g, sc = wl.group, scale_of(wl)
    pg_o, pg_l, pr_o, pr_l = [], [], [], []
    for s in seqs:
        n, qs = wl.kv_lens[s], wl.q_lens[s]
        by_kv = {}
        for i, h in _sample_pairs(rng, wl, s, per_seq):
            by_kv.setdefault(h // g, []).append((i, h))
        for kap, prs in by_kv.items():
            Kh = widen_to_f64(k[ko[s]:ko[s + 1], kap])
            Vh = widen_to_f64(v[ko[s]:ko[s + 1], kap])
            Qr = np.stack([widen_to_f64(q[qo[s] + i, h]) for i, h in prs])
            pos = np.array([n - qs + i for i, _ in prs], dtype=np.int64)
            nb = wl.num_blocks(s)
            for b in sorted({0, nb - 1, int(rng.integers(0, nb))}):
                Ob, Lb = attend_rows(Qr, pos, Kh, Vh, sc, wl.causal, b * wl.block_len, (b + 1) * wl.block_len)
                for i, h in prs:
                    r = partial_row(wl, s, b, kap, i * g + (h - kap * g))
                    pg_o.append(wo[r].cpu().numpy())
                    pg_l.append(float(wlse[r]))
                pr_o.append(Ob)
                pr_l.append(Lb)
    dp = compare(np.stack(pg_o), np.concatenate(pr_o), np.array(pg_l), np.concatenate(pr_l))
    say(f"  sampled partials ({len(pg_o)}): {dp}")
    assert_within(dp, wl.dtype, "sampled partials")


def test_full_small_fp32():
    wl, q, k, v, plan, ws, out, lse = _full("small")
    O, L = attention_ref(widen_to_f64(q), widen_to_f64(k), widen_to_f64(v), wl.kv_lens, wl.q_lens,
                         wl.num_q_heads, wl.num_kv_heads, wl.causal)
    d = compare(out.cpu().numpy(), O, lse.cpu().numpy(), L)
    say(f"  whole output: {d}")
    assert_within(d, wl.dtype, "small fp32 whole output")
    _check_partials_sampled("small", [0], 4)


def test_full_batch8_whole_output():
    _whole("batch8")
    _check_partials_sampled("batch8", range(8), 6)


def test_full_long_whole_output():
    _whole("long")
    _check_partials_sampled("long", [0], 24)


def test_full_lognormal_whole_output():
    wl = get_workload("lognormal")
    _whole("lognormal")
    order = np.argsort(wl.kv_lens)
    seqs = sorted({int(order[0]), int(order[-1]), int(order[len(order) // 2]), int(np.argmax(wl.q_lens)),
                   int(np.argmin(wl.q_lens))})
    _check_partials_sampled("lognormal", seqs, 8)


def test_full_decode_whole_output():
    _whole("decode")
    _check_partials_sampled("decode", [0, 64, 127], 8)


# The mixed batch is compared whole in five parts (its 128 decode sequences, then each
# prefill chunk) so that no single test runs for minutes; the last test combines them.
_MIXED_PARTS = {}


def test_full_mixed_whole_output_decode_part():
    _MIXED_PARTS["decode"] = _whole("mixed", seqs=range(128), what=" (decode sequences)")
    _check_partials_sampled("mixed", [0, 1, 77, 127], 8)


@pytest.mark.parametrize("chunk", range(4))
def test_full_mixed_whole_output_prefill_chunk(chunk):
    _MIXED_PARTS[f"prefill{chunk}"] = _whole("mixed", seqs=[128 + chunk], what=f" (prefill chunk {chunk})")
    if chunk in (0, 3):
        _check_partials_sampled("mixed", [128 + chunk], 8, seed=chunk)


def test_full_mixed_whole_output_combined():
    """Relative L2 over the whole mixed output, from the five parts' sums."""
    if len(_MIXED_PARTS) < 5:
        pytest.skip("needs the five parts of the mixed batch in this session")
    d2 = sum(p.d2 for p in _MIXED_PARTS.values())
    r2 = sum(p.r2 for p in _MIXED_PARTS.values())
    d = Diff(max(p.o_max for p in _MIXED_PARTS.values()), math.sqrt(d2 / r2),
             max(p.lse_max for p in _MIXED_PARTS.values()))
    say(f"  mixed, whole output: {d}")
    assert_within(d, "bfloat16", "mixed whole output")
    _FULL.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("key", ["batch8", "lognormal", "decode"])
def test_full_schedules_agree(key):
    _FULL.clear()
    torch.cuda.empty_cache()
    wl = get_workload(key)
    say(f"[gpu] full-size {wl.name}: static and queue schedules")
    q, k, v = make_qkv(wl, "cuda")
    _schedules_agree(wl, q, k, v)
    del q, k, v
