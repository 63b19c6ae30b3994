"""Host logic: the row kernels' launch plans, checked over every legal width.

Compiles tests/host/launch_plan_check.cpp against the library's launch-plan
header with the host compiler (no GPU, no HIP device code) and runs it: for
every row width of 8..65536 elements, a spread of row counts and of compute
unit counts, each plan must cover its rows with the vectors per thread that the
kernel dispatch instantiates, leave no vector slot wholly idle, and keep the
backward at most two workgroups per compute unit.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM_INCLUDE = "/opt/rocm/include"


def test_launch_plans_cover_every_width(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("needs a host C++ compiler and the ROCm headers")
    exe = str(tmp_path / "launch_plan_check")
    cmd = [cxx, "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(ROOT, 'bloom_bf16_optimizer_amd', 'csrc')}",
           os.path.join(ROOT, "tests", "host", "launch_plan_check.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stdout[-4000:]
    assert "0 failures" in run.stdout
