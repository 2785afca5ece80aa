"""The kernels' single-run test for boundary tiles (visible_run, device_common.h) against
the per-key window predicate, and the plan-free decode's block runs (visible_block_runs)
against the blocks that hold a visible key, on the host: built with hipcc, run without a
GPU."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="needs hipcc")
def test_visible_run_matches_the_window_predicate(tmp_path):
    exe = str(tmp_path / "visible_run_check")
    csrc = os.path.join(ROOT, "structured_sparse_attention_plan_amd", "csrc")
    cmd = [HIPCC if os.path.exists(HIPCC) else "hipcc", "-x", "hip", "--offload-arch=gfx950", "-O2",
           "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(HERE, "visible_run_check.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "with several runs" in r.stdout
    assert "blocks listed in order" in r.stdout
