"""The workgroup -> job maps (XCD remap, its causal interleave, causal tile order) are
permutations: every tile of the grid is computed exactly once.  Built for the host from the
same header the kernels use, and run on the CPU."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_schedule_maps_are_permutations(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "sched_maps"
    p = subprocess.run([hipcc, "--cuda-host-only", "-O2", "-std=c++17", os.path.join(HERE, "sched_maps.hip"),
                        "-o", str(exe)], capture_output=True, text=True)
    assert p.returncode == 0, p.stderr[-2000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr
