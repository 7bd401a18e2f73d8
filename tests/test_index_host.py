"""Host test of the kernels' index arithmetic on malformed cu_seqlens.

Compiles ``tests/index_host_check.cpp`` against the library's
``gdn2_index.h`` with g++ and runs it: sequence ranges clamped into [0, T],
checkpoint slots below T/64 + N, segment indices below the workspace's
segment count, and the slot-to-chunk search, on well-formed and malformed
arrays (no GPU).
"""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_index_helpers_stay_in_bounds(tmp_path):
    exe = tmp_path / "index_host_check"
    src = os.path.join(ROOT, "tests", "index_host_check.cpp")
    inc = os.path.join(ROOT, "linear_attention_rnn_gdn2_amd", "csrc")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-I", inc, src, "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
