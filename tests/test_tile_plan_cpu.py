"""The grouped GEMM's tile schedule (csrc/tile_plan.h) on the host: every tile and K part is
covered exactly once inside the launched grid, split-tail side slots are unique and match the
fixup kernel's enumeration, XCD ranges are balanced, and pair-staged K parts start on even
steps with even lengths (a pair load then never reads past its part's last step, which at the
last part would be past the end of the weight rows). Built with the host compiler; no GPU."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HELPER = os.path.join(ROOT, "tests", "helpers", "tile_plan_check.cpp")
CSRC = os.path.join(ROOT, "sparse_mixture_experts_41_amd", "csrc")


def test_tile_plan_enumeration(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "tile_plan_check")
    subprocess.run([cxx, "-std=c++17", "-O2", "-Wall", "-I", CSRC, HELPER, "-o", exe], check=True,
                   capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
