"""Host check of the kernels' LDS tile layout: the direct tile load, row reads and
transpose reads deliver the promised MFMA operands, and no read instruction has
bank conflicts on a 64-bank LDS (lds_layout_check.cpp, compiled with g++)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
KERNELS = os.path.join(HERE, "..", "masked_long_context_amd", "csrc", "kernels")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_lds_layout(tmp_path):
    exe = tmp_path / "lds_layout_check"
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-I", KERNELS, os.path.join(HERE, "lds_layout_check.cpp"),
                    "-o", str(exe)], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
