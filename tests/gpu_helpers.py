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


class FullOracleCheck:
    """Every byte and every scale of GPU results against the oracle, run on
    the host's cores (``oracle.pool``).

    ``add(name, x, q, s)`` copies the tensor's BF16 bits, codes and scales
    into the current shared block; when a block is full its comparison starts
    in the pool's workers while the next block is filled (the pool holds two
    blocks).  A tensor larger than a block is cut into chunks of whole tile
    rows, which the oracle quantizes independently.  A tensor whose tile rows
    hold more than ``TILE_ROW_VALUES`` values (one scale over a whole tensor,
    say) is compared in two streamed passes: its pieces' partial tile maxima,
    combined by max, then every piece quantized with the full maxima; its
    scales are the oracle's scales of those maxima.  ``finish()`` waits for
    every comparison and raises on the first tensor that differs, naming its
    first differing byte or scale.
    """

    TILE_ROW_VALUES = 1 << 24

    def __init__(self, pool, bm: int, bn: int, what: str = ""):
        self.pool, self.bm, self.bn, self.what = pool, bm, bn, what
        self.cur = 0
        self.items = []
        self.pending = [None] * len(pool.arenas)
        self.failures = []
        self.values = 0
        self.tensors = 0
        pool.arenas[0].reset()
        # values of one chunk: 2 B of x and 1 B of q each, scales and alignment aside
        nbytes = pool.arenas[0].nbytes
        self.capacity = (nbytes - min(64 << 20, nbytes // 8)) // 3
        self.origin = {}    # chunk key -> (tensor name, first row, first tile row)

    def _stage(self, name, x, q, s):
        """Copy one tensor's data into the current block; False if it is full."""
        arena = self.pool.arenas[self.cur]
        xa = arena.array(tuple(x.shape), np.uint16)
        qa = arena.array(tuple(q.shape), np.uint8)
        sa = arena.array(tuple(s.shape), np.float32)
        if xa is None or qa is None or sa is None:
            return False
        for a, t, view_np, view_torch in ((xa, x, np.int16, torch.int16), (qa, q, np.uint8, torch.uint8),
                                          (sa, s, np.float32, torch.float32)):
            if a.size:
                torch.from_numpy(a.view(view_np)).copy_(t.detach().contiguous().view(view_torch))
        self.items.append((name, xa, qa, sa))
        return True

    def _submit(self):
        if self.items:
            self.pending[self.cur] = self.pool.compare_async(self.items, self.bm, self.bn,
                                                             self.pool.arenas[self.cur])
            self.items = []
        self.cur = (self.cur + 1) % len(self.pool.arenas)
        self._collect(self.cur)
        self.pool.arenas[self.cur].reset()

    def _collect(self, k):
        if self.pending[k] is not None:
            for key, (nb, first, ns, first_s) in self.pending[k].get().items():
                if nb or ns:
                    name, r0, t0 = self.origin.get(key, (key, 0, 0))
                    if first is not None:
                        first = (first[0] + r0,) + first[1:]
                    if first_s is not None:
                        first_s = (first_s[0] + t0, first_s[1])
                    self.failures.append((name, (nb, first, ns, first_s)))
            self.pending[k] = None

    def _drain(self):
        """Finish everything in flight; both blocks free, block 0 current."""
        if self.items:
            self._submit()
        for k in range(len(self.pool.arenas)):
            self._collect(k)
            self.pool.arenas[k].reset()
        self.cur = 0

    def _add_one(self, name, x, q, s):
        if not self._stage(name, x, q, s):
            self._submit()
            assert self._stage(name, x, q, s)

    def add(self, name, x, q, s):
        assert tuple(q.shape) == tuple(x.shape)
        M, N = x.shape
        bm, bn = self.bm, self.bn
        self.values += M * N
        self.tensors += 1
        if min(bm, M) * N > self.TILE_ROW_VALUES:
            self._two_pass(name, x, q, s)
            return
        if 3 * M * N + 4 * s.numel() + 1024 <= self.capacity * 3:
            self._add_one(name, x, q, s)
            return
        rows = max(bm, (self.capacity // max(N, 1)) // bm * bm)   # whole tile rows per chunk
        for r0 in range(0, M, rows):
            r1 = min(M, r0 + rows)
            key = f"{name} rows {r0}..{r1 - 1}"
            self.origin[key] = (name, r0, r0 // bm)
            self._add_one(key, x[r0:r1], q[r0:r1], s[r0 // bm:-(-r1 // bm)])

    def _chunks(self, M, N):
        """(r0, r1, c0, c1) chunks of at most ``capacity`` values: whole rows,
        or column runs of one row when a row alone is larger."""
        cap = self.capacity
        if N <= cap:
            rows = cap // N
            return [(r0, min(M, r0 + rows), 0, N) for r0 in range(0, M, rows)]
        return [(r, r + 1, c0, min(N, c0 + cap)) for r in range(M) for c0 in range(0, N, cap)]

    def _two_pass(self, name, x, q, s):
        self._drain()
        bm, bn = self.bm, self.bn
        M, N = x.shape
        TM, TN = -(-M // bm), -(-N // bn)
        chunks = self._chunks(M, N)
        arenas = self.pool.arenas
        amax = np.zeros((TM, TN), dtype=np.float64)
        handles = [None] * len(arenas)

        def copy(arena, t, np_dtype, view_np, view_torch):
            a = arena.array(tuple(t.shape), np_dtype)
            torch.from_numpy(a.view(view_np)).copy_(t.detach().contiguous().view(view_torch))
            return a

        def merge(h):
            if h is not None:
                np.maximum(amax, h.get()[name], out=amax)

        for i, (r0, r1, c0, c1) in enumerate(chunks):      # pass 1: tile maxima
            k = i % len(arenas)
            merge(handles[k])
            arenas[k].reset()
            xa = copy(arenas[k], x[r0:r1, c0:c1], np.uint16, np.int16, torch.int16)
            handles[k] = self.pool.tile_maxima_async([(name, xa, r0, c0, TM, TN)], bm, bn, arenas[k])
        for k in range(len(arenas)):
            merge(handles[k])
            handles[k] = None
        nb, first = 0, None

        def count(h):
            nonlocal nb, first
            if h is not None:
                n1, f1 = h.get()[name]
                nb += n1
                if f1 is not None and (first is None or f1 < first):
                    first = f1

        for i, (r0, r1, c0, c1) in enumerate(chunks):      # pass 2: bytes with the full maxima
            k = i % len(arenas)
            count(handles[k])
            arenas[k].reset()
            xa = copy(arenas[k], x[r0:r1, c0:c1], np.uint16, np.int16, torch.int16)
            qa = copy(arenas[k], q[r0:r1, c0:c1], np.uint8, np.uint8, torch.uint8)
            handles[k] = self.pool.compare_with_maxima_async([(name, xa, qa, r0, c0, amax)], bm, bn,
                                                             arenas[k])
        for k in range(len(arenas)):
            count(handles[k])
            arenas[k].reset()
        s_ref, _ = oracle.blockwise.tile_scales_np(amax)
        bad_s = np.nonzero(scales_bits(s) != scales_bits(s_ref.astype(np.float32)))
        ns = int(bad_s[0].size)
        first_s = (int(bad_s[0][0]), int(bad_s[1][0])) if ns else None
        if nb or ns:
            self.failures.append((name, (nb, first, ns, first_s)))

    def finish(self):
        self._drain()
        if self.failures:
            name, (nb, first, ns, first_s) = self.failures[0]
            msg = (f"{self.what}: {len(self.failures)} tensor(s) differ from the oracle; first {name}: "
                   f"{nb} byte mismatches (first (row, col, got, want) = {first}), "
                   f"{ns} scale mismatches (first tile {first_s})")
            raise AssertionError(msg)
        return self.tensors, self.values
