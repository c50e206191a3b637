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

Every build writes a fingerprint of the code it was built from beside the
library (``libfp8bq.so.sha``): the sources' code with comments and
whitespace runs removed, plus the compiler flags.  ``ensure_built()``
rebuilds when the fingerprint of the sources on disk differs, so a loaded
library always matches the sources next to it.
"""

import hashlib
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "fp8bq.hip")
KERNEL_SOURCES = [os.path.join(HERE, "csrc", "kernels.hpp"), SRC, os.path.join(HERE, "csrc", "div31.hpp")]
DEPS = KERNEL_SOURCES + [os.path.join(ROOT, "include", "fp8bq.h")]
LIB = os.path.join(HERE, "libfp8bq.so")
ARCH = "gfx950"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def flags() -> list:
    return [
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
    ]


def command(out: str = LIB, extra=()) -> list:
    return [hipcc(), *flags(), "-I", os.path.join(ROOT, "include"), *extra, "-o", out, SRC]


def code_only(text: str) -> str:
    """C++ source without comments, whitespace runs collapsed: comment and
    layout edits leave the code, and so the fingerprint, unchanged."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":                     # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def fingerprint(paths, extra: str = "") -> str:
    """16 hex digits of SHA-256 over the files' code (comments excluded)."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
        h.update(b"\0")
    h.update(extra.encode())
    return h.hexdigest()[:16]


def kernel_sha() -> str:
    """Fingerprint of the kernel sources alone (what the committed counter
    profiles are keyed on)."""
    return fingerprint(KERNEL_SOURCES)


def source_sha() -> str:
    """Fingerprint of everything the library is built from: kernel sources,
    the public header and the compiler flags."""
    return fingerprint(DEPS, " ".join(flags()))


def sidecar(lib: str = None) -> str:
    return (lib or LIB) + ".sha"


def built_sha(lib: str = None):
    """Fingerprint recorded by the build that produced ``lib`` (default: the
    in-tree library); None if the record is missing."""
    try:
        with open(sidecar(lib), encoding="utf-8") as f:
            return f.read().strip() or None
    except OSError:
        return None


def build(verbose: bool = False) -> str:
    """Compile the library (always; a stale .so is replaced atomically) and
    record the fingerprint of the sources it was built from."""
    sha = source_sha()
    lib = LIB
    tmp = f"{lib}.tmp{os.getpid()}"  # per process: concurrent builds never share a file
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
    os.replace(tmp, lib)
    side_tmp = f"{sidecar(lib)}.tmp{os.getpid()}"
    with open(side_tmp, "w", encoding="utf-8") as f:
        f.write(sha + "\n")
    os.replace(side_tmp, sidecar(lib))
    return lib


def ensure_built() -> str:
    """Load what is built if it was built from the sources on disk; build
    otherwise (a fresh checkout, an edited kernel, a library with no record)."""
    if not os.path.exists(LIB) or built_sha() != source_sha():
        return build()
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print("source fingerprint", source_sha())
