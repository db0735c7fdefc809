"""The even tile split of the decode kernel, checked on the host.

split_check.cpp includes the same header the kernels use (split.h) and replays every
wave's walk for seeded random batches; it needs hipcc to build but no GPU to run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_351_amd", "csrc")


def test_split_covers_every_tile_once_and_merge_reads_match(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "split_check")
    build = subprocess.run([hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950", f"-I{CSRC}",
                            "-x", "hip", os.path.join(ROOT, "tests", "split_check.cpp"), "-o", exe],
                           capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert run.stdout.startswith("split ok")
