"""Compile-time resource checks of the HIP kernels (CPU only; needs hipcc).

The partial-attention kernel keeps its DMA pipeline in flight only if nothing in its
loop goes through scratch memory: a scratch access is a vector-memory operation, and
waiting for it drains every in-flight stage. Dynamic indexing of per-wave arrays or
register spills put data there, so both must stay at zero.
"""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "split_kv_exact_amd", "csrc")


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not available")


def _resources(src):
    from split_kv_exact_amd.build import EXTRA

    cmd = [_hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *EXTRA.get(src, []), "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", os.devnull, "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    kernels = {}
    cur = None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            kernels[cur] = {}
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)", line)
        if m and cur:
            kernels[cur][m.group(1).strip()] = int(m.group(2))
    return kernels


@pytest.mark.parametrize("src", ["partial_bf16.hip", "partial_mma.hip", "partial_f32.hip", "merge.hip",
                                 "backward_bf16.hip"])
def test_no_scratch_and_no_spills(src):
    ks = _resources(src)
    assert ks, "no kernels reported"
    for name, res in ks.items():
        assert res.get("ScratchSize", 0) == 0, (name, res)
        assert res.get("VGPRs Spill", 0) == 0, (name, res)


@pytest.mark.parametrize("src", ["partial_bf16.hip", "partial_mma.hip"])
def test_partial_kernels_fit_two_waves_per_simd(src):
    for name, res in _resources(src).items():
        assert res.get("VGPRs", 999) + res.get("AGPRs", 0) <= 256, (name, res)
        assert res.get("Occupancy", 2) >= 2, (name, res)
