"""The batch-1 kernel's work split and mailbox tags, checked on the CPU.

tests/plan_check.cpp includes the same header the HIP kernels use (gsi_plan.h) and simulates, for
every site shape of the synthetic workloads and edge shapes, every rank k, both element sizes and
both grid sizes, where each 16-byte chunk of a block's LDS region is copied from and where phase A,
the gate piece and phase B read it; then it checks the mailbox tag arithmetic against an explicit
model of the mailbox words.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plan_and_tags(tmp_path):
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "plan_check"
    src = os.path.join(ROOT, "tests", "plan_check.cpp")
    inc = os.path.join(ROOT, "gated_rank_linear_amd", "csrc")
    r = subprocess.run([cxx, "-O2", "-std=c++17", "-Wall", "-I", inc, src, "-o", str(exe)], capture_output=True,
                       text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "passed" in r.stdout
