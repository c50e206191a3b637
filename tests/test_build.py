"""The loaded library is tied to the sources it was built from: every build
records a fingerprint of the sources' code and the compiler flags beside the
.so, and ensure_built() rebuilds when the sources on disk differ."""

import os
import shutil
import sys

import pytest

from fp8_blockwise_weight_amd import build


@pytest.fixture
def sandbox(tmp_path, monkeypatch):
    """A copy of the sources and a stand-in compiler that only writes the
    output file, so the test runs in milliseconds and needs no hipcc."""
    srcs = []
    for p in build.DEPS:
        dst = tmp_path / os.path.basename(p)
        shutil.copy(p, dst)
        srcs.append(str(dst))
    lib = str(tmp_path / "libfp8bq.so")
    calls = []

    def fake_command(out, extra=()):
        calls.append(out)
        return [sys.executable, "-c", f"open({out!r}, 'w').write('lib')"]

    monkeypatch.setattr(build, "DEPS", srcs)
    monkeypatch.setattr(build, "KERNEL_SOURCES", [srcs[1], srcs[0], srcs[2]])
    monkeypatch.setattr(build, "LIB", lib)
    monkeypatch.setattr(build, "command", fake_command)
    return srcs, lib, calls


def test_rebuild_follows_the_sources(sandbox, monkeypatch):
    srcs, lib, calls = sandbox
    kernels = next(p for p in srcs if p.endswith("kernels.hpp"))
    build.ensure_built()                       # nothing built yet
    assert len(calls) == 1 and os.path.exists(lib)
    assert build.built_sha(lib) == build.source_sha()
    build.ensure_built()                       # same sources: load as is
    assert len(calls) == 1
    with open(kernels, "a", encoding="utf-8") as f:
        f.write("\n// a comment changes no code\n/* nor does this */\n")
    build.ensure_built()
    assert len(calls) == 1
    with open(kernels, "a", encoding="utf-8") as f:
        f.write("\nstatic constexpr int fp8bq_edit_marker = 1;\n")
    old = build.built_sha(lib)
    assert old != build.source_sha()
    build.ensure_built()                       # code edit: rebuilt
    assert len(calls) == 2 and build.built_sha(lib) == build.source_sha() != old
    os.remove(build.sidecar(lib))              # a library with no record is rebuilt
    build.ensure_built()
    assert len(calls) == 3
    monkeypatch.setattr(build, "flags", lambda: ["-O2"])   # other compiler flags: rebuilt
    build.ensure_built()
    assert len(calls) == 4


def test_header_edit_rebuilds(sandbox):
    srcs, lib, calls = sandbox
    header = next(p for p in srcs if p.endswith("fp8bq.h"))
    build.ensure_built()
    with open(header, "a", encoding="utf-8") as f:
        f.write("\n#define FP8BQ_EDIT_MARKER 1\n")
    build.ensure_built()
    assert len(calls) == 2


def test_in_tree_library_matches_sources():
    """The session start (conftest) ensured the build: the library in the
    tree carries the fingerprint of the sources in the tree."""
    assert os.path.exists(build.LIB)
    assert build.built_sha() == build.source_sha()
