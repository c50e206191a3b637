"""Host logic on the CPU: the multiply-and-shift division (csrc/div31.hpp)
that the dequantization kernel uses for its row and tile indices, compiled
with g++ and checked against the C division operator (exhaustively over all
numerators below 2^31 for five divisors, and at edge and random numerators
for every divisor up to 65536 and 200,000 random larger ones)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_div31_matches_integer_division(tmp_path):
    exe = tmp_path / "div31_check"
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "fp8_blockwise_weight_amd", "csrc"),
           os.path.join(ROOT, "tests", "c", "div31_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "div31 ok (exhaustive divisors included)" in res.stdout
