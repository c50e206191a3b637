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
