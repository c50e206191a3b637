"""The C header and library from a plain C99 program (gcc), CPU only: every
call made there is rejected by argument checks before any device access."""

import os
import shutil
import subprocess

import pytest

import fp8_blockwise_weight_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="fake-pointer validation program runs only on machines without a visible GPU")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_c99_client_compiles_links_and_validates(tmp_path):
    fq.load_library()  # the library must be built
    libdir = os.path.dirname(fq.LIB_PATH)
    exe = tmp_path / "abi_check"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
           "-L", libdir, "-lfp8bq", f"-Wl,-rpath,{libdir}", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi ok" in res.stdout
