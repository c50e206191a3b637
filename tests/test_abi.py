"""C-ABI library: loads, exports every declared symbol, and rejects every bad
argument before touching a device (CPU only: no call here reaches a kernel).

Calls with fake pointer values are all built so that an argument check
rejects them; none of them may ever pass validation.
"""

import ctypes
import os
import re

import pytest

import fp8_blockwise_weight_amd as fq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bq.h")

# These calls pass fake device addresses; they are only ever run where no GPU
# is visible, so even a wrongly accepted call cannot reach a kernel.
pytestmark = pytest.mark.skipif(
    __import__("torch").cuda.device_count() > 0,
    reason="fake-pointer validation tests run only on machines without a visible GPU")

INVALID = fq.ERR_INVALID_ARGUMENT
WORKSPACE = fq.ERR_WORKSPACE

# Fake, never dereferenced addresses (16-byte aligned, far apart).
X = 0x10_0000_0000
Q = 0x20_0000_0000
S = 0x30_0000_0000
W = 0x40_0000_0000


@pytest.fixture(scope="module")
def lib():
    return fq.load_library()


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(fp8bq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(fq.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(5):
        assert lib.fp8bq_status_string(code)
    assert lib.fp8bq_status_string(99) == b"unknown status"
    assert lib.fp8bq_last_hip_error() == 0


def test_workspace_bytes(lib):
    # groups of up to 512 tensors carry their table in the kernel arguments
    for n in (-3, 0, 1, 7, 252, 256, 512):
        assert lib.fp8bq_many_workspace_bytes(n) == 0
    for n in (513, 4096, 20000):
        b = lib.fp8bq_many_workspace_bytes(n)
        assert b >= 64 * n + 8 * (n + 1) and b % 256 == 0


@pytest.mark.parametrize("args", [
    (X, -1, 128, 128, 128, Q, S),          # negative M
    (X, 128, -1, 128, 128, Q, S),          # negative N
    (X, 128, 128, 0, 128, Q, S),           # bm < 1
    (X, 128, 128, 128, 0, Q, S),           # bn < 1
    (X, 128, 128, -5, 128, Q, S),
    (None, 128, 128, 128, 128, Q, S),      # null x
    (X, 128, 128, 128, 128, None, S),      # null q
    (X, 128, 128, 128, 128, Q, None),      # null scale
    (X + 1, 128, 128, 128, 128, Q, S),     # x not 2-byte aligned
    (X, 128, 128, 128, 128, Q, S + 2),     # scale not 4-byte aligned
    (X, 128, 128, 128, 128, X + 100, S),   # q overlaps x
    (X, 128, 128, 128, 128, Q, X + 4),     # scale overlaps x
    (X, 128, 128, 128, 128, Q, Q + 16),    # scale overlaps q
    (X, 1 << 31, 8, 128, 128, Q, S),       # M too large
    (X, 8, 1 << 31, 128, 128, Q, S),       # N too large
    (X, 1 << 20, 1 << 20, 1, 1, Q, S),     # 2^40 tiles
])
def test_quantize_rejects(lib, args):
    x, M, N, bm, bn, q, s = args
    assert lib.fp8bq_quantize(x, M, N, bm, bn, q, s, None) == INVALID


@pytest.mark.parametrize("M,N", [(0, 128), (128, 0), (0, 0)])
def test_quantize_empty_is_ok_without_device(lib, M, N):
    # Empty input: nothing to do, no device is touched (null pointers allowed).
    assert lib.fp8bq_quantize(None, M, N, 128, 128, None, None, None) == fq.OK


def _entries(rows):
    arr = (fq.TensorEntry * len(rows))()
    for i, (x, q, s, M, N) in enumerate(rows):
        arr[i].x, arr[i].q, arr[i].scale_inv, arr[i].M, arr[i].N = x, q, s, M, N
    return arr


def test_quantize_many_rejects(lib):
    good = _entries([(X, Q, S, 256, 256)])
    f = lib.fp8bq_quantize_many
    assert f(good, -1, 128, 128, W, 0, None) == INVALID             # count < 0
    assert f(None, 1, 128, 128, W, 0, None) == INVALID              # null list
    assert f(good, 1, 0, 128, W, 0, None) == INVALID                # bm < 1
    assert f(good, 1, 128, 0, W, 0, None) == INVALID                # bn < 1
    # more than 512 entries need a workspace (each entry its own fake slab)
    many = _entries([(X + i * 0x100000, Q + i * 0x100000, S + i * 0x1000, 256, 256)
                     for i in range(600)])
    need = lib.fp8bq_many_workspace_bytes(600)
    assert need > 0
    assert f(many, 600, 128, 128, None, need, None) == WORKSPACE    # null workspace
    assert f(many, 600, 128, 128, W, need - 1, None) == WORKSPACE   # too small
    assert f(many, 600, 128, 128, W + 8, need, None) == WORKSPACE   # misaligned
    # one bad entry anywhere rejects the whole call
    bad = _entries([(X, Q, S, 256, 256), (X + 0x1000000, None, S + 0x1000, 4, 4)])
    assert f(bad, 2, 128, 128, W, lib.fp8bq_many_workspace_bytes(2), None) == INVALID
    bad = _entries([(X, Q, S, 256, 256), (X, Q, S, -1, 4)])
    assert f(bad, 2, 128, 128, W, lib.fp8bq_many_workspace_bytes(2), None) == INVALID
    bad = _entries([(X, X + 64, S, 256, 256)])                     # q overlaps x
    assert f(bad, 1, 128, 128, W, need, None) == INVALID


def test_quantize_many_noalloc_rejects(lib):
    """The workspace-free grouped call checks everything before any HIP call:
    lists beyond FP8BQ_NOALLOC_MAX_TENSORS are refused (nothing read past the
    count check), and the usual argument errors."""
    f = lib.fp8bq_quantize_many_noalloc
    good = _entries([(X, Q, S, 256, 256)])
    assert fq.NOALLOC_MAX_TENSORS == 16384
    assert f(good, fq.NOALLOC_MAX_TENSORS + 1, 128, 128, None) == WORKSPACE
    assert f(good, -1, 128, 128, None) == INVALID
    assert f(None, 1, 128, 128, None) == INVALID
    assert f(good, 1, 0, 128, None) == INVALID
    assert f(good, 1, 128, 0, None) == INVALID
    assert f(None, 0, 128, 128, None) == fq.OK
    empty = _entries([(None, None, None, 0, 4096), (None, None, None, 7, 0)])
    assert f(empty, 2, 128, 128, None) == fq.OK
    bad = _entries([(X, Q, S, 256, 256), (X + 0x1000000, None, S + 0x1000, 4, 4)])
    assert f(bad, 2, 128, 128, None) == INVALID
    many = _entries([(X + i * 0x100000, Q + i * 0x100000, S + i * 0x1000, 256, 256)
                     for i in range(599)] + [(X, X + 64, S, 256, 256)])   # the last: q overlaps x
    assert f(many, 600, 128, 128, None) == INVALID
    with pytest.raises(ValueError):
        fq.quantize_many_noalloc([None] * (fq.NOALLOC_MAX_TENSORS + 1),
                                 [None] * (fq.NOALLOC_MAX_TENSORS + 1))


def _shards(rows):
    arr = (fq.ShardEntry * len(rows))()
    for e, (x, q, a, sc, M, N, rp, cp) in zip(arr, rows):
        e.x, e.q, e.amax, e.scale_inv, e.M, e.N, e.row_phase, e.col_phase = x, q, a, sc, M, N, rp, cp
    return arr


def test_shard_entry_layout_matches_header():
    # fp8bq_shard: four pointers, two int64, two int32 -> 56 bytes on LP64
    assert ctypes.sizeof(fq.ShardEntry) == 56


def test_shard_many_rejects(lib):
    """Grouped shard calls check every entry as the single calls do, before
    anything is enqueued (no device needed to reject)."""
    A = S + 0x100000
    good = [(X, Q, A, S, 256, 256, 64, 0)]
    for f, quant in ((lib.fp8bq_tile_amax_many, False), (lib.fp8bq_quantize_amax_many, True)):
        assert f(_shards(good), -1, 128, 128, None) == INVALID           # count < 0
        assert f(None, 1, 128, 128, None) == INVALID                     # null list
        assert f(_shards(good), 1, 0, 128, None) == INVALID              # bm < 1
        assert f(_shards(good), 1, 128, 0, None) == INVALID              # bn < 1
        for bad in [(X, Q, A, S, -1, 256, 0, 0),                         # negative M
                    (X, Q, A, S, 256, 256, 128, 0),                      # row phase >= bm
                    (X, Q, A, S, 256, 256, 0, -1),                       # negative column phase
                    (None, Q, A, S, 256, 256, 0, 0),                     # null x
                    (X, Q, None, S, 256, 256, 0, 0),                     # null amax
                    (X + 1, Q, A, S, 256, 256, 0, 0),                    # x not 2-byte aligned
                    (X, Q, A + 2, S, 256, 256, 0, 0),                    # amax not 4-byte aligned
                    (X, Q, X + 8, S, 256, 256, 0, 0)]:                   # amax overlaps x
            # one bad entry after a good one rejects the whole call
            assert f(_shards(good + [bad]), 2, 128, 128, None) == INVALID, (quant, bad)
        if quant:
            for bad in [(X, None, A, S, 256, 256, 0, 0),                 # null q
                        (X, Q, A, None, 256, 256, 0, 0),                 # null scale_inv
                        (X, X + 64, A, S, 256, 256, 0, 0),               # q overlaps x
                        (X, Q, A, A + 4, 256, 256, 0, 0)]:               # amax partly overlaps scale
                assert f(_shards(good + [bad]), 2, 128, 128, None) == INVALID, bad


def _rows(rows):
    arr = (fq.RowShardEntry * len(rows))()
    for e, (x, q, sc, ta, ba, M, N, rp) in zip(arr, rows):
        e.x, e.q, e.scale_inv, e.top_amax, e.bottom_amax, e.M, e.N, e.row_phase = x, q, sc, ta, ba, M, N, rp
    return arr


def test_row_shard_entry_layout_matches_header():
    # fp8bq_row_shard: five pointers, two int64, two int32 -> 64 bytes on LP64
    assert ctypes.sizeof(fq.RowShardEntry) == 64


def test_row_shards_reject(lib):
    """Both row-shard calls check every entry as a whole before anything is
    enqueued: ranges, null pointers, alignment, overlaps within an entry
    (an edge's maxima may be its own scale row), and the workspace of the
    whole-tile parts."""
    # 300 x 256 rows at row phase 64 of [128,128]: 64 top rows, 108 bottom
    # rows, 3 local tile rows x 2 tile columns; maxima in their scale rows
    first, last = S, S + 4 * 2 * 2
    good = (X, Q, S, first, last, 300, 256, 64)
    A = S + 0x100000
    begin = lambda arr, n, bm=128, bn=128, ws=None, wsb=0: lib.fp8bq_row_shards_begin(
        arr, n, bm, bn, ws, wsb, None, None)
    finish = lambda arr, n, bm=128, bn=128: lib.fp8bq_row_shards_finish(arr, n, bm, bn, None)
    for f in (begin, finish):
        assert f(_rows([good]), -1) == INVALID                          # count < 0
        assert f(None, 1) == INVALID                                     # null list
        assert f(_rows([good]), 1, bm=0) == INVALID                      # bm < 1
        assert f(_rows([good]), 1, bn=0) == INVALID                      # bn < 1
        assert f(None, 0) == fq.OK
        for bad in [(X, Q, S, first, last, -1, 256, 64),                 # negative M
                    (X, Q, S, first, last, 300, 1 << 31, 64),            # N beyond 32 bits
                    (X, Q, S, first, last, 300, 256, 128),               # row phase >= bm
                    (X, Q, S, first, last, 300, 256, -1),                # negative row phase
                    (None, Q, S, first, last, 300, 256, 64),             # null x
                    (X, None, S, first, last, 300, 256, 64),             # null q
                    (X, Q, None, first, last, 300, 256, 64),             # null scale_inv
                    (X + 1, Q, S, first, last, 300, 256, 64),            # x not 2-byte aligned
                    (X, Q, S + 2, first, last, 300, 256, 64),            # scale_inv not 4-byte aligned
                    (X, Q, S, None, last, 300, 256, 64),                 # top rows, no top maxima
                    (X, Q, S, first, None, 300, 256, 64),                # bottom rows, no bottom maxima
                    (X, Q, S, A + 2, last, 300, 256, 64),                # maxima not 4-byte aligned
                    (X, X + 64, S, first, last, 300, 256, 64),           # q overlaps x
                    (X, Q, X + 8, first, last, 300, 256, 64),            # scale_inv overlaps x
                    (X, Q, S, Q + 16, last, 300, 256, 64),               # top maxima overlap q
                    (X, Q, S, X, last, 300, 256, 64),                    # top maxima overlap x
                    (X, Q, S, S + 4, last, 300, 256, 64),                # inside scale_inv, not its row
                    (X, Q, S, first, first, 300, 256, 64),               # bottom maxima in the first row
                    (X, Q, S, A, A + 4, 300, 256, 64)]:                  # the two maxima overlap
            assert f(_rows([good, bad]), 2) == INVALID, bad
    # maxima beside scale_inv, and a shard with no edges (phase 0, whole tile
    # rows): no maxima needed -- still refused here only through the workspace
    many = _rows([good] * 600)
    assert begin(many, 600) == WORKSPACE                                 # > 512 whole-tile parts
    need = lib.fp8bq_many_workspace_bytes(600)
    assert begin(many, 600, ws=W, wsb=need - 1) == WORKSPACE
    assert begin(many, 600, ws=W + 8, wsb=need) == WORKSPACE             # not 16-byte aligned
    # entries with M == 0 or N == 0 (any maxima) and lists of them need no device
    empty = _rows([(None, None, None, None, None, 0, 256, 5), (None, None, None, None, None, 300, 0, 7)])
    assert begin(empty, 2) == fq.OK
    assert finish(empty, 2) == fq.OK


def test_row_shard_edges_rejects(lib):
    t, b = ctypes.c_int64(), ctypes.c_int64()
    f = lib.fp8bq_row_shard_edges
    assert f(10, 128, 0, ctypes.byref(t), ctypes.byref(b)) == fq.OK
    assert f(-1, 128, 0, ctypes.byref(t), ctypes.byref(b)) == INVALID
    assert f(1 << 31, 128, 0, ctypes.byref(t), ctypes.byref(b)) == INVALID
    assert f(10, 0, 0, ctypes.byref(t), ctypes.byref(b)) == INVALID
    assert f(10, 128, 128, ctypes.byref(t), ctypes.byref(b)) == INVALID
    assert f(10, 128, -1, ctypes.byref(t), ctypes.byref(b)) == INVALID
    assert f(10, 128, 0, None, ctypes.byref(b)) == INVALID


def test_shard_many_empty_is_ok_without_device(lib):
    empty = _shards([(None, None, None, None, 0, 8, 0, 0), (None, None, None, None, 8, 0, 0, 0)])
    assert lib.fp8bq_tile_amax_many(empty, 2, 128, 128, None) == fq.OK
    assert lib.fp8bq_quantize_amax_many(empty, 2, 128, 128, None) == fq.OK
    assert lib.fp8bq_tile_amax_many(None, 0, 128, 128, None) == fq.OK


def test_quantize_many_empty_is_ok_without_device(lib):
    assert lib.fp8bq_quantize_many(None, 0, 128, 128, None, 0, None) == fq.OK
    empty = _entries([(None, None, None, 0, 4096), (None, None, None, 7, 0)])
    assert lib.fp8bq_quantize_many(empty, 2, 128, 128, W, lib.fp8bq_many_workspace_bytes(2),
                                   None) == fq.OK


def test_encode_rejects(lib):
    assert lib.fp8bq_encode_e4m3(X, Q, -1, None) == INVALID
    assert lib.fp8bq_encode_e4m3(None, Q, 10, None) == INVALID
    assert lib.fp8bq_encode_e4m3(X, None, 10, None) == INVALID
    assert lib.fp8bq_encode_e4m3(X + 2, Q, 10, None) == INVALID
    assert lib.fp8bq_encode_e4m3(X, X + 8, 10, None) == INVALID     # overlap
    assert lib.fp8bq_encode_e4m3(None, None, 0, None) == fq.OK


def test_resident_wait_limit(lib):
    """The wait limit of the one-scale-per-tensor kernel: range checked, no
    device touched, and the Python setter round-trips."""
    assert lib.fp8bq_set_resident_wait_us(-1) == INVALID
    assert lib.fp8bq_set_resident_wait_us(2 ** 40 + 1) == INVALID
    assert lib.fp8bq_set_resident_wait_us(0) == fq.OK
    assert lib.fp8bq_set_resident_wait_us(2 ** 40) == fq.OK
    assert lib.fp8bq_set_resident_wait_us(2000) == fq.OK
    with pytest.raises(fq.Fp8bqError):
        fq.set_resident_wait_us(-5)
    fq.set_resident_wait_us(2000)
    assert lib.fp8bq_last_hip_error() == 0


def test_dequantize_rejects(lib):
    f = lib.fp8bq_dequantize
    assert f(Q, S, -1, 128, 128, 128, X, 0, None) == INVALID        # negative M
    assert f(Q, S, 128, 128, 0, 128, X, 0, None) == INVALID         # bm < 1
    assert f(Q, S, 128, 128, 128, 128, X, 2, None) == INVALID       # unknown out dtype
    assert f(None, S, 128, 128, 128, 128, X, 0, None) == INVALID    # null q
    assert f(Q, None, 128, 128, 128, 128, X, 0, None) == INVALID    # null scale
    assert f(Q, S, 128, 128, 128, 128, None, 0, None) == INVALID    # null out
    assert f(Q, S + 1, 128, 128, 128, 128, X, 0, None) == INVALID   # scale misaligned
    assert f(Q, S, 128, 128, 128, 128, X + 1, 1, None) == INVALID   # bf16 out misaligned
    assert f(Q, S, 128, 128, 128, 128, X + 2, 0, None) == INVALID   # fp32 out misaligned
    assert f(Q, S, 128, 128, 128, 128, Q + 64, 0, None) == INVALID  # out overlaps q
    assert f(Q, S, 128, 128, 128, 128, S - 64, 0, None) == INVALID  # out overlaps scale
    assert f(None, None, 0, 128, 128, 128, None, 0, None) == fq.OK


def test_dq_entry_layout_matches_header():
    # fp8bq_dq_tensor: three pointers, two int64 -> 40 bytes on LP64
    assert ctypes.sizeof(fq.DqEntry) == 40


def test_dequantize_many_rejects(lib):
    """Grouped dequantization: every entry is checked as the single call
    checks it, before anything is enqueued (no device is touched here)."""
    f = lib.fp8bq_dequantize_many

    def table(*entries):
        arr = (fq.DqEntry * len(entries))()
        for i, e in enumerate(entries):
            arr[i] = fq.DqEntry(*e)
        return arr

    good = (Q, S, X, 128, 128)
    assert f(table(good), -1, 128, 128, 0, None) == INVALID          # negative count
    assert f(None, 2, 128, 128, 0, None) == INVALID                  # null list
    assert f(table(good), 1, 0, 128, 0, None) == INVALID             # bm < 1
    assert f(table(good), 1, 128, 128, 3, None) == INVALID           # unknown out dtype
    assert f(table(good, (Q, S, X + 2, 128, 128)), 2, 128, 128, 0, None) == INVALID  # out misaligned
    assert f(table(good, (Q, S, Q + 64, 128, 128)), 2, 128, 128, 0, None) == INVALID  # out overlaps q
    assert f(table(good, (None, S, X, 128, 128)), 2, 128, 128, 1, None) == INVALID  # null q
    assert f(table(good, (Q, S, X, -1, 128)), 2, 128, 128, 0, None) == INVALID  # negative M
    assert f(None, 0, 128, 128, 0, None) == fq.OK                    # nothing to do
    assert f(table((None, None, None, 0, 128), (None, None, None, 7, 0)), 2, 128, 128, 1, None) == fq.OK
    assert lib.fp8bq_last_hip_error() == 0


def test_shard_calls_reject(lib):
    ta, qa = lib.fp8bq_tile_amax, lib.fp8bq_quantize_amax
    A = 0x50_0000_0000
    assert ta(X, 128, 128, 128, 128, 128, 0, A, None) == INVALID     # row phase >= bm
    assert ta(X, 128, 128, 128, 128, 0, -1, A, None) == INVALID      # negative phase
    assert ta(X, 128, 128, 0, 128, 0, 0, A, None) == INVALID         # bm < 1
    assert ta(None, 128, 128, 128, 128, 0, 0, A, None) == INVALID
    assert ta(X, 128, 128, 128, 128, 0, 0, None, None) == INVALID
    assert ta(X, 128, 128, 128, 128, 0, 0, A + 2, None) == INVALID   # amax misaligned
    assert ta(X, 128, 128, 128, 128, 0, 0, X + 64, None) == INVALID  # amax overlaps x
    assert ta(None, 0, 128, 128, 128, 0, 0, None, None) == fq.OK
    assert qa(X, 128, 128, 128, 128, 0, 128, A, Q, S, None) == INVALID   # col phase >= bn
    assert qa(X, 128, 128, 128, 128, 0, 0, None, Q, S, None) == INVALID
    assert qa(X, 128, 128, 128, 128, 0, 0, A, None, S, None) == INVALID
    assert qa(X, 128, 128, 128, 128, 0, 0, A, Q, None, None) == INVALID
    # amax [8, 8] floats at S, scale_inv at S + 4: the two ranges partly overlap
    assert qa(X, 1024, 1024, 128, 128, 0, 0, S + 0, Q, S + 4, None) == INVALID
    assert qa(X, 128, 128, 128, 128, 0, 0, A, X + 2, S, None) == INVALID      # q overlaps x
    assert qa(None, 5, 0, 128, 128, 0, 0, None, None, None, None) == fq.OK


def test_python_block_size_checks():
    with pytest.raises(ValueError):
        fq.block_shape(None)
    with pytest.raises(ValueError):
        fq.block_shape((0, 128))
    assert fq.block_shape([128, 128]) == (128, 128)
    assert fq.scale_shape(4097, 11008, 128, 128) == (33, 86)


def test_python_rejects_cpu_tensor():
    import torch

    with pytest.raises(TypeError):
        fq.quantize(torch.zeros(4, 4, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        fq.quantize(torch.zeros(4, 4, dtype=torch.float32))


def test_entry_layout_matches_header():
    # fp8bq_tensor: three pointers then two int64 -> 40 bytes on LP64
    assert ctypes.sizeof(fq.TensorEntry) == 40


def test_python_output_checks():
    """Caller-supplied outputs are checked before any library call."""
    import torch

    cpu = torch.device("cpu")
    q = torch.empty((4, 8), dtype=torch.uint8)
    s = torch.empty((1, 1), dtype=torch.float32)
    fq._check_outputs((q, s), 4, 8, 128, 128, cpu)                     # exact match passes
    with pytest.raises(ValueError):
        fq._check_outputs((torch.empty((4, 9), dtype=torch.uint8), s), 4, 8, 128, 128, cpu)
    with pytest.raises(ValueError):
        fq._check_outputs((q, torch.empty((3, 1))), 4, 8, 2, 128, cpu)  # scale must be (2, 1)
    fq._check_outputs((q, torch.empty((2, 1))), 4, 8, 2, 128, cpu)
    with pytest.raises(TypeError):
        fq._check_outputs((torch.empty((4, 8), dtype=torch.int16), s), 4, 8, 128, 128, cpu)
    with pytest.raises(TypeError):
        fq._check_outputs((q, s.to(torch.float64)), 4, 8, 128, 128, cpu)
    with pytest.raises(ValueError):
        fq._check_outputs((torch.empty((8, 4), dtype=torch.uint8).t(), s), 4, 8, 128, 128, cpu)


def test_group_outputs_layout():
    """Outputs a grouped call allocates: per tensor, a contiguous [M, N] e4m3
    view and a [TM, TN] fp32 view, in input order, pairwise disjoint, empty
    shapes included (host logic, CPU tensors)."""
    import torch

    for shapes in ([(5, 8), (3, 16), (0, 8), (7, 8), (2, 0), (130, 16), (1, 24)],
                   [(5, 16), (0, 16), (130, 16), (1, 16)]):      # several row lengths, or one
        _check_group_outputs(torch, shapes)


def _check_group_outputs(torch, shapes):
    xs = [torch.empty(sh, dtype=torch.bfloat16) for sh in shapes]
    entries, views = fq._plan_outputs([tuple(x.shape) for x in xs], [x.data_ptr() for x in xs],
                                      4, 8, torch.device("cpu"))
    assert len(entries) == ctypes.sizeof(fq.TensorEntry) * len(xs)
    outs = list(zip(*views()))
    table = (fq.TensorEntry * len(xs)).from_buffer(entries)
    spans = []
    for x, (q, s), e in zip(xs, outs, table):
        assert q.shape == x.shape and q.dtype == torch.float8_e4m3fn and q.is_contiguous()
        assert tuple(s.shape) == fq.scale_shape(*x.shape, 4, 8)
        assert s.dtype == torch.float32 and s.is_contiguous()
        # the table the library receives points at exactly these views
        assert (e.x or 0, e.M, e.N) == (x.data_ptr(), x.shape[0], x.shape[1])
        if x.numel():
            assert (e.q, e.scale_inv) == (q.data_ptr(), s.data_ptr())
        for t in (q, s):
            if t.numel():
                spans.append((t.data_ptr(), t.data_ptr() + t.numel() * t.element_size()))
    spans.sort()
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
