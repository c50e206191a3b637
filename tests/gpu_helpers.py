"""Helpers for the GPU parity tests: move data to the host and compare the
HIP path with the CPU oracle (full tensors, sampled tiles, or all scales)."""

import numpy as np
import torch

import oracle


def bits_np(x: torch.Tensor) -> np.ndarray:
    """BF16 tensor (any device) -> uint16 numpy array of its bit patterns."""
    return x.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def codes_np(q: torch.Tensor) -> np.ndarray:
    return q.detach().view(torch.uint8).cpu().numpy()


def scales_bits(s) -> np.ndarray:
    if isinstance(s, torch.Tensor):
        s = s.detach().cpu().numpy()
    return np.ascontiguousarray(s, dtype=np.float32).view(np.uint32)


def assert_matches_oracle(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, bm: int, bn: int,
                          what: str = ""):
    """Whole tensor: GPU bytes and scales equal the oracle's, bit for bit."""
    q_ref, s_ref = oracle.quantize(bits_np(x), bm, bn)
    q_got = codes_np(q)
    assert s.shape == s_ref.shape, (what, tuple(s.shape), s_ref.shape)
    bad_s = np.nonzero(scales_bits(s) != scales_bits(s_ref))
    assert bad_s[0].size == 0, (what, "scale mismatch at tiles", list(zip(*bad_s))[:5])
    bad = np.nonzero(q_got != q_ref)
    if bad[0].size:
        r, c = bad[0][0], bad[1][0]
        raise AssertionError(f"{what}: {bad[0].size} byte mismatches; first at ({r},{c}): "
                             f"got {q_got[r, c]:#04x} want {q_ref[r, c]:#04x}")


def tile_amax_gpu(x: torch.Tensor, bm: int, bn: int) -> np.ndarray:
    """Exact per-tile max |x| (float64 [TM, TN]) computed on the GPU by torch."""
    M, N = x.shape
    TM, TN = -(-M // bm), -(-N // bn)
    a = x.abs()
    if TM * bm != M or TN * bn != N:
        pad = torch.zeros((TM * bm, TN * bn), dtype=x.dtype, device=x.device)
        pad[:M, :N] = a
        a = pad
    m = a.view(TM, bm, TN, bn).amax(dim=(1, 3))
    return m.float().cpu().numpy().astype(np.float64)


def assert_scales_match_oracle(x: torch.Tensor, s: torch.Tensor, bm: int, bn: int, what=""):
    """Every scale of a tensor of any size: the oracle's scale function applied
    to the exact per-tile maximum (taken on the GPU by torch)."""
    amax = tile_amax_gpu(x, bm, bn)
    s_ref, _ = oracle.blockwise.tile_scales_np(amax)
    got = scales_bits(s)
    want = scales_bits(s_ref.astype(np.float32))
    bad = np.nonzero(got != want)
    assert bad[0].size == 0, (what, "scale mismatches", bad[0].size)


def assert_tiles_match_oracle(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, bm: int, bn: int,
                              tiles, what=""):
    """Sampled tiles: the oracle run on each tile alone (tile independence)
    equals the GPU bytes and scale of that tile."""
    M, N = x.shape
    s_host = s.detach().cpu().numpy()
    for ti, tj in tiles:
        r0, r1 = ti * bm, min(M, (ti + 1) * bm)
        c0, c1 = tj * bn, min(N, (tj + 1) * bn)
        xt = bits_np(x[r0:r1, c0:c1].contiguous())
        q_ref, s_ref = oracle.quantize(xt, bm, bn)
        assert s_ref.shape == (1, 1)
        assert scales_bits(s_host[ti:ti + 1, tj:tj + 1])[0, 0] == scales_bits(s_ref)[0, 0], \
            (what, ti, tj)
        got = codes_np(q[r0:r1, c0:c1].contiguous())
        assert np.array_equal(got, q_ref), (what, "tile", ti, tj)


def sample_tiles(M, N, bm, bn, k, seed):
    """k random tiles plus the four corner tiles (edges included)."""
    TM, TN = -(-M // bm), -(-N // bn)
    rng = np.random.default_rng(seed)
    tiles = {(0, 0), (TM - 1, TN - 1), (0, TN - 1), (TM - 1, 0)}
    for _ in range(k):
        tiles.add((int(rng.integers(TM)), int(rng.integers(TN))))
    return sorted(tiles)


def assert_properties_gpu(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, bm: int, bn: int,
                          what=""):
    """Invariants that hold at any size, checked on the GPU with torch:
    no NaN codes (I8); every tile whose max is >= eps holds a +-448 code and
    no code above it (I1); all-zero tiles hold only zero codes (I2); signs
    of q follow signs of x (I5)."""
    codes = q.view(torch.uint8)
    assert not bool(((codes == 0x7F) | (codes == 0xFF)).any()), (what, "NaN code")
    mag = (codes & 0x7F).to(torch.int16)
    M, N = x.shape
    TM, TN = -(-M // bm), -(-N // bn)
    if TM * bm != M or TN * bn != N:
        pad = torch.zeros((TM * bm, TN * bn), dtype=torch.int16, device=x.device)
        pad[:M, :N] = mag
        mag = pad
    tile_max = mag.view(TM, bm, TN, bn).amax(dim=(1, 3))
    eps32 = float(np.float32(oracle.EPS))
    amax = torch.from_numpy(tile_amax_gpu(x, bm, bn)).to(x.device)
    big = amax >= eps32
    assert bool((tile_max[big] == 0x7E).all()), (what, "tile max code")
    assert bool((tile_max[amax == 0] == 0).all()), (what, "zero tile code")
    xs = x.view(torch.int16) < 0
    qs = (codes & 0x80) != 0
    assert bool((xs == qs).all()), (what, "sign")
