"""The GEMM split plans' workgroup mapping, checked on the host with the library's own
code (tests/split_mapping_harness.cpp, compiled with hipcc; no GPU is used)."""

import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "nf4_weight_streamed_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_balanced_and_tail_split_mapping(tmp_path):
    exe = tmp_path / "split_mapping"
    subprocess.run([HIPCC, "-std=c++17", "-O1", "-x", "hip", "--offload-arch=gfx950", "-I", CSRC,
                    os.path.join(HERE, "split_mapping_harness.cpp"), "-o", str(exe)],
                   check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok"), res.stdout
