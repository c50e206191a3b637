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


def _rocm_tool(*parts):
    path = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), *parts)
    return path if os.path.exists(path) else None


@pytest.mark.skipif(_rocm_tool("bin", "hipcc") is None or _rocm_tool("llvm", "bin", "clang") is None,
                    reason="ROCm hipcc/clang not available")
def test_c99_client_under_host_address_and_ub_sanitizers(tmp_path):
    """The same program against a library whose host code is built with
    AddressSanitizer and UndefinedBehaviorSanitizer (device code unchanged):
    every argument check runs instrumented, and any sanitizer report fails."""
    from fp8_blockwise_weight_amd import build as fb

    lib = tmp_path / "libfp8bq.so"
    cmd = fb.command(str(lib), extra=("-O1", "-g",
                                      "-Xarch_host", "-fsanitize=address",
                                      "-Xarch_host", "-fsanitize=undefined",
                                      "-Xarch_host", "-fno-sanitize-recover=all",
                                      "-Xarch_host", "-fno-omit-frame-pointer"))
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    exe = tmp_path / "abi_check_san"
    client = [_rocm_tool("llvm", "bin", "clang"), "-std=c99", "-Wall", "-Wextra", "-Werror",
              "-pedantic", "-g", "-fno-sanitize-recover=all",
              "-fsanitize=address,undefined",
              "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c", "abi_check.c"),
              "-L", str(tmp_path), "-lfp8bq", f"-Wl,-rpath,{tmp_path}", "-o", str(exe)]
    subprocess.run(client, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=23",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "abi ok" in res.stdout
    assert "Sanitizer" not in res.stderr, res.stderr
