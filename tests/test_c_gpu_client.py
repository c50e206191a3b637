"""The library from a native C++ program on the GPU, with no Python in the
process (tests/c/gpu_client.cpp): a direct quantize, a grouped call captured
in a HIP graph and replayed, two grouped calls of the entry point that
allocates nothing (over 512 entries), two row shards whose shared tile row's
maxima are exchanged on a second stream between the two row-shard calls,
and a dequantization, checked here against the CPU oracle.  The client is
host code only and builds with g++ in seconds."""

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import fp8_blockwise_weight_amd as fq
import oracle
from fp8_blockwise_weight_amd import workloads as wl
from gpu_helpers import bits_np

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def client(tmp_path_factory, gpu_lib):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    libdir = os.path.dirname(fq.LIB_PATH)
    exe = tmp_path_factory.mktemp("client") / "gpu_client"
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "gpu_client.cpp"),
           "-L", libdir, "-lfp8bq", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}", "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr[-3000:]
    return exe


def _c5(M, N):
    return [sp for sp in wl.c5() if (sp.M, sp.N) == (M, N)][0]


CASES = [
    ("c1 256x256", lambda: wl.materialize(wl.c1()[0], "cuda:0"), (128, 128)),
    ("1000x3000 [128,128]", lambda: wl.materialize(_c5(1000, 3000), "cuda:0"), (128, 128)),
    ("77x128 [1,128]", lambda: wl.materialize(_c5(77, 128), "cuda:0"), (1, 128)),
    ("1000x3000 [64,64]", lambda: wl.materialize(_c5(1000, 3000), "cuda:0"), (64, 64)),
    ("99x37 [5,3]", lambda: (torch.randn((99, 37), generator=torch.Generator().manual_seed(7))
                             * 0.05).to(torch.bfloat16).cuda(), (5, 3)),
]


@pytest.mark.parametrize("name,make,block", CASES, ids=[c[0] for c in CASES])
def test_native_client_matches_oracle(client, tmp_path, name, make, block):
    x = make()
    bits = bits_np(x)
    M, N = bits.shape
    bm, bn = block
    src = tmp_path / "x.bf16"
    bits.astype("<u2").tofile(src)
    prefix = tmp_path / "out"
    _say("native client", name)
    res = subprocess.run([str(client), str(src), str(M), str(N), str(bm), str(bn), str(prefix)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "gpu client ok" in res.stdout
    TM, TN = fq.scale_shape(M, N, bm, bn)
    q = np.fromfile(f"{prefix}.q", dtype=np.uint8).reshape(M, N)
    s = np.fromfile(f"{prefix}.s", dtype="<f4").reshape(TM, TN)
    deq = np.fromfile(f"{prefix}.deq", dtype="<f4").reshape(M, N)
    q_ref, s_ref = oracle.quantize(bits, bm, bn)
    assert np.array_equal(s.view(np.uint32), np.asarray(s_ref, dtype=np.float32).view(np.uint32)), name
    assert np.array_equal(q, q_ref), name
    deq_ref = oracle.dequantize(q_ref, s_ref, bm, bn, "f32").astype(np.float32)
    assert np.array_equal(deq.view(np.uint32), deq_ref.view(np.uint32)), name
