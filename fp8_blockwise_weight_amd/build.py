"""Build libfp8bq.so in-tree with hipcc for gfx950.

Usage: ``python -m fp8_blockwise_weight_amd.build`` (or ``build()``).

Flags that matter for bit-exactness:
  -ffp-contract=off                            no fused multiply-adds
  -fhip-fp32-correctly-rounded-divide-sqrt     IEEE binary32 division
  -fno-gpu-flush-denormals-to-zero             keep denormals
  (no -ffast-math or -funsafe-math-optimizations anywhere)
``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the compiler from
emitting packed fp32 instructions; the host pass warns that it does not
know the feature, which is harmless.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "fp8bq.hip")
DEPS = [SRC, os.path.join(HERE, "csrc", "kernels.hpp"), os.path.join(HERE, "csrc", "div31.hpp"),
        os.path.join(ROOT, "include", "fp8bq.h")]
LIB = os.path.join(HERE, "libfp8bq.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def command(out: str = LIB, extra=()) -> list:
    return [
        hipcc(),
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-shared",
        "-ffp-contract=off",
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        "-fno-gpu-flush-denormals-to-zero",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall",
        "-I", os.path.join(ROOT, "include"),
        *extra,
        "-o", out,
        SRC,
    ]


def build(verbose: bool = False) -> str:
    """Compile the library (always; a stale .so is replaced atomically)."""
    tmp = f"{LIB}.tmp{os.getpid()}"  # per process: concurrent builds never share a file
    cmd = command(tmp)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln and ln.strip()]
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


def ensure_built() -> str:
    """Build the library only when none is there (a fresh checkout); an
    existing build is loaded as it is."""
    if not os.path.exists(LIB):
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
