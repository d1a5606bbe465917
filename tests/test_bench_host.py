"""Host-side pieces of bench.py and the byte / flop accounting (CPU only)."""

import os
import shutil
import subprocess
import sys

import bench
from split_kv_exact_amd import metrics as M
from workloads import Workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hash_ignores_comments_only(tmp_path):
    csrc = os.path.join(ROOT, "split_kv_exact_amd", "csrc")
    for f in bench.KERNEL_SOURCES:
        shutil.copy(os.path.join(csrc, f), tmp_path / f)
    base = bench._kernel_sha(str(tmp_path))
    assert base == bench._kernel_sha(csrc)
    p = tmp_path / "partial_mma.hip"
    text = p.read_text()
    p.write_text("// a new comment\n" + text.replace("\n", "\n  \n", 3) + "/* trailing\n block */\n")
    assert bench._kernel_sha(str(tmp_path)) == base
    assert "constexpr int NST = 4;" in text
    p.write_text(text.replace("constexpr int NST = 4;", "constexpr int NST = 3;"))
    assert bench._kernel_sha(str(tmp_path)) != base


def test_traffic_record_needs_current_sources_and_the_same_workload(tmp_path, monkeypatch):
    """A committed counter record is used only on the sources and the workload (shape and
    block size, both in the name) it was taken on."""
    import json

    (tmp_path / "profiles").mkdir()
    rec = {"kernel_sha": "abc", "workload": "mix_b8192", "hbm_bytes_per_launch": 123}
    (tmp_path / "profiles" / "traffic_mix.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_kernel_sha", lambda csrc=None: "abc")
    assert bench._traffic("mix", "mix_b8192") == 123
    assert bench._traffic("mix", "mix_b4096") is None
    assert bench._traffic("other", "mix_b8192") is None
    monkeypatch.setattr(bench, "_kernel_sha", lambda csrc=None: "def")
    assert bench._traffic("mix", "mix_b8192") is None


def test_byte_and_flop_accounting_by_hand():
    # Two causal sequences, bf16, Hq = 4, Hkv = 2 (g = 2), D = 8, B = 4.
    wl = Workload(name="t", dtype="bfloat16", kv_lens=(6, 3), q_lens=(2, 3), num_q_heads=4, num_kv_heads=2,
                  head_dim=8, block_len=4, num_workers=3)
    # Visible pairs: sequence 0 rows at positions 4, 5 see 5 + 6 keys; sequence 1 rows at
    # positions 0, 1, 2 see 1 + 2 + 3 keys.
    assert M.visible_pairs(wl) == 17
    assert M.flops(wl) == 4 * 8 * 4 * 17
    kv = 2 * 9 * 2 * 8 * 2  # K and V: 9 tokens x 2 heads x 8 dims x 2 bytes
    q = 5 * 4 * 8 * 2
    out = 5 * 4 * (8 + 1) * 4
    assert M.kv_bytes(wl) == kv and M.q_bytes(wl) == q and M.out_bytes(wl) == out
    assert M.effective_bytes(wl) == kv + q + out
    # Partial rows: sequence 0 has 2 blocks x 2 KV heads x (2 queries x g 2), sequence 1
    # one block x 2 x (3 x 2).
    assert M.partial_rows(wl) == 2 * 2 * 4 + 1 * 2 * 6
    # Every unit reads its block's query rows: blocks x q x Hq elements. bf16 inputs keep
    # their partials as fp16 elements with an fp32 (LSE, scale) pair: 8 * 2 + 8 bytes a row.
    assert M.partial_kernel_bytes(wl) == kv + (2 * 2 * 4 + 1 * 3 * 4) * 8 * 2 + 28 * (8 * 2 + 8)
    assert M.merge_kernel_bytes(wl) == 28 * (8 * 2 + 8) + out
    assert M.partial_traffic_bytes(wl) == 2 * 28 * (8 * 2 + 8)
    f32 = Workload(name="t", dtype="float32", kv_lens=(6, 3), q_lens=(2, 3), num_q_heads=4, num_kv_heads=2,
                   head_dim=8, block_len=4, num_workers=3)
    assert M.partial_traffic_bytes(f32) == 2 * 28 * 9 * 4
