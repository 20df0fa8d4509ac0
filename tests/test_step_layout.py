"""Host replay of the fused step kernel's gather rule and LDS layout: the
checker (step_layout_check.cpp) is built with g++ from the kernel's own
layout header and run for every block-table width and candidate count."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "learned_block_sparse_tok_amd", "csrc")


def test_step_gather_rule_and_layout(tmp_path):
    exe = tmp_path / "step_layout_check"
    subprocess.check_call(["g++", "-std=c++17", "-O2", "-Wall", "-I", CSRC,
                           os.path.join(HERE, "step_layout_check.cpp"), "-o", str(exe)])
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok")
