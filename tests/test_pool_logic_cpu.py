"""The block pool's state machine (pool_core.h, the code stream_pool.cpp runs on HIP)
driven by a host engine on the CPU (tests/pool_harness.cpp): the order of copies and
reads carried by its events, data integrity, and the error states."""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "nf4_weight_streamed_amd", "csrc")
CXX = shutil.which("g++")


@pytest.mark.skipif(CXX is None, reason="g++ not available")
def test_pool_state_machine_on_a_host_engine(tmp_path):
    exe = tmp_path / "pool_harness"
    subprocess.run([CXX, "-std=c++17", "-O1", "-Wall", "-I", CSRC, os.path.join(HERE, "pool_harness.cpp"), "-o",
                    str(exe)], check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok"), res.stdout
