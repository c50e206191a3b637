"""The multi-process oracle runner: slabs of whole tile rows run in worker
processes give exactly the whole-tensor oracle output, and the comparison
finds and places planted mismatches."""

import numpy as np
import pytest

import oracle
from oracle.pool import OraclePool, default_workers


def _bits(rng, M, N):
    x = (rng.standard_normal((M, N)) * 0.02).astype(np.float32)
    x[rng.random((M, N)) < 0.001] *= 200.0
    if M:
        x[M // 3] = 0.0                               # a zero row
    return (x.view(np.uint32) >> 16).astype(np.uint16)  # truncation: any BF16 patterns do


CASES = [((300, 520), (128, 128)), ((257, 384), (64, 64)), ((77, 128), (1, 128)),
         ((1000, 264), (5, 3)), ((0, 128), (128, 128)), ((129, 1), (128, 128))]


@pytest.fixture(scope="module")
def pool():
    # tiny slabs: every tensor is cut into many slabs, some with ragged ends
    with OraclePool(64 << 20, workers=3, slab_values=3000) as p:
        yield p


def _load(pool, rng):
    pool.arena.reset()
    items, refs = [], []
    for i, ((M, N), (bm, bn)) in enumerate(CASES):
        x = pool.arena.array((M, N), np.uint16)
        x[...] = _bits(rng, M, N)
        q_ref, s_ref = oracle.quantize(x, bm, bn)
        q = pool.arena.array((M, N), np.uint8)
        s = pool.arena.array(s_ref.shape, np.float32)
        items.append((i, x, q, s))
        refs.append((q_ref, s_ref))
    return items, refs


def test_quantize_equals_whole_tensor_oracle(pool):
    rng = np.random.default_rng(1)
    items, refs = _load(pool, rng)
    for (i, x, q, s), ((M, N), (bm, bn)), (q_ref, s_ref) in zip(items, CASES, refs):
        q[...] = 0xAA
        s[...] = -1.0
        pool.quantize([(i, x, q, s)], bm, bn)
        assert np.array_equal(q, q_ref), i
        assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), i


def test_compare_finds_planted_mismatches(pool):
    rng = np.random.default_rng(2)
    items, refs = _load(pool, rng)
    for (i, x, q, s), ((M, N), (bm, bn)), (q_ref, s_ref) in zip(items, CASES, refs):
        q[...] = q_ref
        s[...] = s_ref
        res = pool.compare([(i, x, q, s)], bm, bn)
        assert res[i] == (0, None, 0, None), i
        if M * N == 0:
            continue
        # one wrong byte in the last row, one wrong scale in the last tile row
        r, c = M - 1, N // 2
        q[r, c] ^= 0x01
        tm, tn = s.shape[0] - 1, s.shape[1] - 1
        s[tm, tn] = np.nextafter(s[tm, tn], np.float32(1))
        nb, first, ns, first_s = pool.compare([(i, x, q, s)], bm, bn)[i]
        assert (nb, ns) == (1, 1), i
        assert first == (r, c, int(q[r, c]), int(q_ref[r, c])), i
        assert first_s == (tm, tn), i


def test_default_workers_is_bounded():
    assert 1 <= default_workers() <= 16


def test_full_check_streams_blocks_and_reports():
    """The streaming checker the GPU tests use, fed CPU tensors: tensors pass
    through several small blocks (both blocks reused), a correct set passes,
    and a planted wrong byte is reported with its tensor and place."""
    import torch

    from gpu_helpers import FullOracleCheck

    rng = np.random.default_rng(3)
    shapes = [(300, 256), (129, 640), (64, 1024), (257, 128), (0, 128), (500, 264)]
    data = []
    for M, N in shapes:
        bits = _bits(rng, M, N) if M else np.zeros((0, N), np.uint16)
        q_ref, s_ref = oracle.quantize(bits, 128, 128)
        x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
        data.append((x, torch.from_numpy(q_ref.copy()), torch.from_numpy(s_ref.copy())))
    with OraclePool(600_000, workers=2, slab_values=20000, arenas=2) as pool:
        chk = FullOracleCheck(pool, 128, 128, "cpu set")
        for i, (x, q, s) in enumerate(data * 3):
            chk.add(f"t{i}", x, q, s)
        assert chk.finish() == (18, 3 * sum(M * N for M, N in shapes))
        bad_q = data[5][1].clone()
        bad_q[499, 7] ^= 0x80
        chk = FullOracleCheck(pool, 128, 128, "cpu set")
        for i, (x, q, s) in enumerate(data):
            chk.add(f"t{i}", x, bad_q if i == 5 else q, s)
        with pytest.raises(AssertionError, match=r"t5: 1 byte mismatches \(first \(row, col, got, want\) = \(499, 7"):
            chk.finish()


@pytest.mark.parametrize("shape,block,arena", [((300, 520), (300, 520), 60_000),  # one tile, row chunks
                                               ((1, 5000), (1, 5000), 12_000),    # one tile, column chunks
                                               ((37, 700), (16, 300), 60_000),    # tiles larger than pieces
                                               ((3, 4000), (1, 4000), 30_000)])   # one tile per row
def test_two_pass_equals_whole_tensor_oracle(shape, block, arena):
    """Tensors whose tiles exceed a piece go through the two passes (partial
    maxima of pieces combined by max, then quantize with the full maxima):
    equal to the oracle on the whole tensor, and planted wrong bytes and
    scales are found and placed in the tensor's coordinates."""
    import torch

    from gpu_helpers import FullOracleCheck

    rng = np.random.default_rng(sum(shape))
    M, N = shape
    bm, bn = block
    bits = _bits(rng, M, N)
    q_ref, s_ref = oracle.quantize(bits, bm, bn)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    with OraclePool(arena, workers=2, slab_values=700, arenas=2) as pool:
        chk = FullOracleCheck(pool, bm, bn, "two-pass")
        chk.TILE_ROW_VALUES = 600
        assert chk.capacity < M * N           # several chunks as well
        chk.add("t", x, torch.from_numpy(q_ref.copy()), torch.from_numpy(s_ref.copy()))
        assert chk.finish() == (1, M * N)
        bad_q = torch.from_numpy(q_ref.copy())
        bad_q[M - 1, N - 3] ^= 0x01
        bad_s = torch.from_numpy(s_ref.copy())
        bad_s[-1, -1] = bad_s[-1, -1] * 2
        chk = FullOracleCheck(pool, bm, bn, "two-pass")
        chk.TILE_ROW_VALUES = 600
        chk.add("t", x, bad_q, bad_s)
        want = int(bad_q[M - 1, N - 3])
        tm, tn = s_ref.shape
        with pytest.raises(AssertionError, match=rf"t: 1 byte mismatches \(first \(row, col, got, want\) = "
                                                 rf"\({M - 1}, {N - 3}, {want}, {int(q_ref[M - 1, N - 3])}\)\), "
                                                 rf"1 scale mismatches \(first tile \({tm - 1}, {tn - 1}\)\)"):
            chk.finish()


def test_tensors_larger_than_a_block_are_cut_into_tile_rows():
    """A tensor larger than one shared block is compared in chunks of whole
    tile rows; a wrong byte in a later chunk is reported at its tensor row."""
    import torch

    from gpu_helpers import FullOracleCheck

    rng = np.random.default_rng(9)
    M, N, bm, bn = 700, 256, 64, 128
    bits = _bits(rng, M, N)
    q_ref, s_ref = oracle.quantize(bits, bm, bn)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    with OraclePool(120_000, workers=2, slab_values=5000, arenas=2) as pool:
        chk = FullOracleCheck(pool, bm, bn, "chunks")
        assert chk.capacity < M * N
        q = torch.from_numpy(q_ref.copy())
        q[650, 100] ^= 0x04
        chk.add("big", x, q, torch.from_numpy(s_ref.copy()))
        with pytest.raises(AssertionError, match=r"big: 1 byte mismatches \(first \(row, col, got, want\) = \(650, 100"):
            chk.finish()
