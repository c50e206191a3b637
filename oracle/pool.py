"""The oracle on many host cores (test infrastructure only).

Runs ``oracle.quantize`` over slabs of whole tile rows in a pool of worker
processes, so full-size weight sets (billions of values) can be compared
with the GPU output byte for byte, and the oracle can be timed on the
host's cores.  Nothing here computes anything of the method itself: every
byte and scale comes from ``oracle.blockwise.quantize``.

Why slabs of whole tile rows give the whole tensor's result: the blockwise
cast (page "fp8_kernel.py — FP8 量化内核", section 2) computes each tile from
that tile's elements alone, and ``quantize`` walks the tensor one tile row at
a time; a slab that starts and ends on tile-row boundaries therefore holds
exactly the tiles, bytes and scales of those rows of the whole tensor.

Tiles too large for one slab (one scale over a whole tensor, say) take two
passes over pieces of the tile: ``oracle.tile_amax`` gives each piece's
partial maxima, which combine by max into the tiles' maxima, and
``oracle.quantize_with_amax`` quantizes each piece with them.  The pages'
cast takes one maximum per tile, so cutting a tile, taking the max of the
pieces' maxima and scaling every piece by the tile's reciprocal reproduces
the whole tile (the oracle's own pins check that equivalence on shards cut
anywhere).

Data sits in one block of shared host memory (an anonymous memory file that
the workers map through /proc): the main process copies inputs and outputs
into arrays carved from it, workers map the same block and read and write
in place, and only small descriptors cross the process boundary.  Workers
are started with the "spawn" method and import only numpy and this package.
"""

import mmap
import multiprocessing as mp
import os
import time

import numpy as np

from .blockwise import local_grid, quantize, quantize_with_amax, tile_amax, tile_grid

MAX_WORKERS = 16          # one GPU's share of a host's cores
_ALIGN = 256


def default_workers() -> int:
    """Cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


class Arena:
    """One block of shared host memory handed out as numpy arrays (bump
    allocation; ``reset`` frees all of them at once)."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.fd = os.memfd_create("fp8bq-oracle-arena")
        os.ftruncate(self.fd, self.nbytes)
        self.path = f"/proc/{os.getpid()}/fd/{self.fd}"
        self.map = mmap.mmap(self.fd, self.nbytes)
        self.buf = np.frombuffer(self.map, dtype=np.uint8)
        self.base = self.buf.__array_interface__["data"][0]
        self.top = 0

    def array(self, shape, dtype) -> np.ndarray:
        """A new array in the block, or None when it does not fit."""
        dtype = np.dtype(dtype)
        size = int(np.prod(shape, dtype=np.int64)) * dtype.itemsize
        off = -(-self.top // _ALIGN) * _ALIGN
        if off + size > self.nbytes:
            return None
        self.top = off + size
        return self.buf[off:off + size].view(dtype).reshape(shape)

    def descriptor(self, arr: np.ndarray, row0: int = 0, row1: int = None):
        """(offset, shape, dtype) of rows [row0, row1) of an array of the block."""
        row1 = arr.shape[0] if row1 is None else row1
        if arr.size == 0 or row0 == row1:
            return (0, (row1 - row0,) + arr.shape[1:], arr.dtype.str)
        off = arr.__array_interface__["data"][0] - self.base
        if not (arr.flags.c_contiguous and 0 <= off and off + arr.nbytes <= self.nbytes):
            raise ValueError("not a contiguous array of this block")
        row_bytes = int(np.prod(arr.shape[1:], dtype=np.int64)) * arr.dtype.itemsize
        return (off + row0 * row_bytes, (row1 - row0,) + arr.shape[1:], arr.dtype.str)

    def reset(self) -> None:
        self.top = 0

    def close(self) -> None:
        self.buf = None
        try:
            self.map.close()
        except BufferError:   # arrays still held by the caller keep the mapping
            pass
        os.close(self.fd)


# ------------------------------------------------------------------ worker side

_MAPS = {}


def _view(path, desc) -> np.ndarray:
    m = _MAPS.get(path)
    if m is None:
        with open(path, "r+b") as f:
            m = _MAPS[path] = mmap.mmap(f.fileno(), 0)
    off, shape, dtype = desc
    n = int(np.prod(shape, dtype=np.int64)) * np.dtype(dtype).itemsize
    return np.frombuffer(m, dtype=np.uint8, count=n, offset=off).view(dtype).reshape(shape)


def _compare_slab(task):
    """Oracle on one slab of whole tile rows, compared with the given bytes
    and scales.  Returns (slab id, byte mismatches, first one as (row, col,
    got, want), scale mismatches, first one as (tile row, tile col))."""
    path, key, xd, qd, sd, bm, bn = task
    x, q, s = _view(path, xd), _view(path, qd), _view(path, sd)
    q_ref, s_ref = quantize(x, bm, bn)
    bad = np.nonzero(q != q_ref)
    first = None
    if bad[0].size:
        r, c = int(bad[0][0]), int(bad[1][0])
        first = (r, c, int(q[r, c]), int(q_ref[r, c]))
    bad_s = np.nonzero(s.view(np.uint32) != s_ref.view(np.uint32))
    first_s = (int(bad_s[0][0]), int(bad_s[1][0])) if bad_s[0].size else None
    return key, int(bad[0].size), first, int(bad_s[0].size), first_s


def _quantize_slab(task):
    """Oracle on one slab, its bytes and scales written in place."""
    path, key, xd, qd, sd, bm, bn = task
    q_ref, s_ref = quantize(_view(path, xd), bm, bn)
    _view(path, qd)[...] = q_ref
    _view(path, sd)[...] = s_ref
    return key


def _piece(path, xd, c0, c1):
    return _view(path, xd)[:, c0:c1]


def _amax_piece(task):
    """Partial tile maxima of one piece (rows of a slab, columns c0..c1) at
    its tile phase.  Returns (key, first tile row, first tile column, maxima)."""
    path, key, xd, c0, c1, bm, bn, rp, cp, t0, u0 = task
    return key, t0, u0, tile_amax(_piece(path, xd, c0, c1), bm, bn, rp, cp)


def _compare_piece_amax(task):
    """One piece quantized with its tiles' full maxima, compared with the
    given bytes.  Returns (key, (row, col) of the piece in the tensor,
    mismatches, first (row, col, got, want) inside the piece)."""
    path, key, xd, qd, c0, c1, bm, bn, rp, cp, origin, amax = task
    q_ref, _ = quantize_with_amax(_piece(path, xd, c0, c1), bm, bn, amax, rp, cp)
    q = _view(path, qd)[:, c0:c1]
    bad = np.nonzero(q != q_ref)
    first = None
    if bad[0].size:
        r, c = int(bad[0][0]), int(bad[1][0])
        first = (r, c, int(q[r, c]), int(q_ref[r, c]))
    return key, origin, int(bad[0].size), first


def _ping(path):
    return _view(path, (0, (1,), "|u1")).shape


# ------------------------------------------------------------------ main side

class OraclePool:
    """A pool of oracle workers and the shared block they work in.

    ``items`` below are (key, x, q, s) with x the [M, N] uint16 BF16 bit
    patterns, q the [M, N] uint8 codes and s the [TM, TN] float32 scales,
    all arrays of ``self.arena``.
    """

    def __init__(self, arena_bytes: int, workers: int = None, slab_values: int = None,
                 arenas: int = 1):
        self.workers = workers or default_workers()
        self.slab_values = slab_values
        self.arenas = [Arena(arena_bytes) for _ in range(arenas)]
        self.arena = self.arenas[0]
        self.pool = mp.get_context("spawn").Pool(self.workers)
        # every worker up and able to map the blocks before anything is timed
        paths = [a.path for a in self.arenas] * (4 * self.workers)
        self.pool.map(_ping, paths, chunksize=1)

    def close(self) -> None:
        self.pool.terminate()
        self.pool.join()
        for a in self.arenas:
            a.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _tasks(self, items, bm, bn, arena=None):
        """Split every item into slabs of whole tile rows, sized so that the
        pool gets several slabs per worker and no slab is large."""
        arena = arena or self.arena
        total = sum(x.size for _, x, _, _ in items)
        target = self.slab_values or min(max(total // (8 * self.workers), 1 << 20), 1 << 24)
        tasks = []
        for key, x, q, s in items:
            M, N = x.shape
            TM, TN = tile_grid(M, N, bm, bn)
            if q.shape != (M, N) or s.shape != (TM, TN):
                raise ValueError(f"{key}: output shapes {q.shape}, {s.shape} do not fit {x.shape}")
            if M == 0 or N == 0:
                continue
            per = max(1, target // (bm * N))                # tile rows per slab
            for t0 in range(0, TM, per):
                t1 = min(TM, t0 + per)
                r0, r1 = t0 * bm, min(M, t1 * bm)
                tasks.append((arena.path, (key, r0, t0),
                              arena.descriptor(x, r0, r1), arena.descriptor(q, r0, r1),
                              arena.descriptor(s, t0, t1), bm, bn))
        return tasks

    def compare_async(self, items, bm: int, bn: int, arena=None):
        """Start comparing every byte and scale of every item with the
        oracle; ``.get()`` of the result gives what ``compare`` returns."""
        keys = [key for key, *_ in items]
        res = self.pool.map_async(_compare_slab, self._tasks(items, bm, bn, arena), chunksize=1)
        return _Comparison(keys, res)

    def compare(self, items, bm: int, bn: int, arena=None):
        """Every byte and scale of every item against the oracle.  Returns
        {key: (byte mismatches, first, scale mismatches, first)} with the
        first mismatch in the item's own row / tile-row numbering."""
        return self.compare_async(items, bm, bn, arena).get()

    def _pieces(self, arena, x, r0, c0, bm, bn):
        """Pieces of an array holding rows r0.. and columns c0.. of a tensor:
        row groups of whole rows of the array, or column runs of single rows
        when a row alone exceeds the piece size.  Yields (descriptor of the
        row group, first and last column in the array, row phase, column
        phase, first tile row, first tile column, row offset in the array)."""
        M, N = x.shape
        target = self.slab_values or min(max(x.size // (8 * self.workers), 1 << 20), 1 << 24)
        rows = max(1, target // max(N, 1))
        cols = N if rows > 1 or N <= target else target
        for a in range(0, M, rows):
            b = min(M, a + rows)
            desc = arena.descriptor(x, a, b)
            for ca in range(0, N, cols):
                cb = min(N, ca + cols)
                g, h = r0 + a, c0 + ca
                yield desc, ca, cb, g % bm, h % bn, g // bm, h // bn, a

    def tile_maxima_async(self, items, bm: int, bn: int, arena=None):
        """Start the partial tile maxima of every item, where an item is
        (key, x, r0, c0, TM, TN): the part of a tensor from row r0 and column
        c0 on, whose full tile grid is TM x TN.  ``.get()`` gives {key:
        float64 [TM, TN]} with the maxima over the items' elements (zero
        where an item holds none of a tile)."""
        arena = arena or self.arena
        tasks, shapes = [], {}
        for key, x, r0, c0, TM, TN in items:
            shapes[key] = (TM, TN)
            for desc, ca, cb, rp, cp, t0, u0, _ in self._pieces(arena, x, r0, c0, bm, bn):
                tasks.append((arena.path, key, desc, ca, cb, bm, bn, rp, cp, t0, u0))
        res = self.pool.map_async(_amax_piece, tasks, chunksize=1)
        return _Maxima(shapes, res)

    def compare_with_maxima_async(self, items, bm: int, bn: int, arena=None):
        """Start comparing the bytes of every item, (key, x, q, r0, c0, amax):
        the part of a tensor from row r0 and column c0 on and its codes,
        quantized with the tensor's full tile maxima ``amax`` [TM, TN].
        ``.get()`` gives {key: (byte mismatches, first (row, col, got, want)
        in the tensor's coordinates)}."""
        arena = arena or self.arena
        tasks = []
        for key, x, q, r0, c0, amax in items:
            for desc, ca, cb, rp, cp, t0, u0, a in self._pieces(arena, x, r0, c0, bm, bn):
                rows = desc[1][0]
                TMl, TNl = local_grid(rows, cb - ca, bm, bn, rp, cp)
                tasks.append((arena.path, key, desc, arena.descriptor(q, a, a + rows), ca, cb, bm, bn,
                              rp, cp, (r0 + a, c0 + ca),
                              np.ascontiguousarray(amax[t0:t0 + TMl, u0:u0 + TNl])))
        res = self.pool.map_async(_compare_piece_amax, tasks, chunksize=1)
        return _PieceComparison([key for key, *_ in items], res)

    def quantize(self, items, bm: int, bn: int, arena=None) -> float:
        """Quantize every item with the oracle into its q and s arrays;
        returns the wall time in seconds (the pool's work alone)."""
        tasks = self._tasks(items, bm, bn, arena)
        t0 = time.perf_counter()
        for _ in self.pool.imap_unordered(_quantize_slab, tasks, chunksize=1):
            pass
        return time.perf_counter() - t0


class _Comparison:
    """Slab results of one comparison, merged per item on ``get``."""

    def __init__(self, keys, res):
        self.keys, self.res = keys, res

    def get(self):
        out = {key: [0, None, 0, None] for key in self.keys}
        for (key, r0, t0), nb, first, ns, first_s in self.res.get():
            rec = out[key]
            if nb:
                rec[0] += nb
                cand = (first[0] + r0,) + first[1:]
                rec[1] = cand if rec[1] is None or cand < rec[1] else rec[1]
            if ns:
                rec[2] += ns
                cand = (first_s[0] + t0, first_s[1])
                rec[3] = cand if rec[3] is None or cand < rec[3] else rec[3]
        return {k: tuple(v) for k, v in out.items()}


class _Maxima:
    """Partial maxima of pieces, combined per item by max on ``get``."""

    def __init__(self, shapes, res):
        self.shapes, self.res = shapes, res

    def get(self):
        out = {key: np.zeros(shape, dtype=np.float64) for key, shape in self.shapes.items()}
        for key, t0, u0, m in self.res.get():
            dst = out[key][t0:t0 + m.shape[0], u0:u0 + m.shape[1]]
            np.maximum(dst, m, out=dst)
        return out


class _PieceComparison:
    """Byte mismatches of pieces, merged per item on ``get``."""

    def __init__(self, keys, res):
        self.keys, self.res = keys, res

    def get(self):
        out = {key: [0, None] for key in self.keys}
        for key, (r0, c0), nb, first in self.res.get():
            if nb:
                rec = out[key]
                rec[0] += nb
                cand = (first[0] + r0, first[1] + c0) + first[2:]
                rec[1] = cand if rec[1] is None or cand < rec[1] else rec[1]
        return {k: tuple(v) for k, v in out.items()}
