"""Blockwise FP8 quantization, plain and slow (test infrastructure only).

Follows the blockwise cast on the documentation page "fp8_kernel.py — FP8
量化内核" (verl/utils/kernel/fp8_kernel.py):

* section 1 (unified entry point): an [M, N] high-precision matrix and a
  [BLOCK_M, BLOCK_N] block size go in; the FP8 data and a descale per block
  come out;
* section 2 (Triton implementation): one program per block loads the block,
  takes the largest magnitude floored at ``eps``, divides it by the FP8
  maximum to get the stored scale, multiplies the block by the reciprocal of
  that scale, clamps to the FP8 range and stores the cast values and the
  scale.

Readings where the page is silent (each is listed in the design notes):

* compute precision is float32; both divisions are correctly rounded float32
  divisions and the reciprocal is taken of the rounded scale (``1/s``, not
  ``448/amax``);
* ``eps`` is 1e-10 rounded to float32 (the page names ``eps`` without a value);
* ``fp8_min``/``fp8_max`` are -448/+448, the e4m3fn range;
* the maximum runs over the whole tile; edge tiles take it over their valid
  elements only and nothing outside [M, N] exists;
* the cast rounds to nearest even (e4m3fn has no infinities; the clamp keeps
  every value finite and in range);
* the descale is a float32 [ceil(M/bm), ceil(N/bn)] row-major array, and
  dequantization is ``decode(q) * s``;
* non-finite input is outside the contract: the oracle raises on it.
"""

import math

import numpy as np

from .e4m3fn import decode_np, encode, encode_np
from .fp32 import bf16_bits_to_f64, bf16_bits_to_float, fl32

E4M3_MAX = 448.0
EPS = 1e-10            # floor for the tile maximum; rounded to float32 before use


def tile_grid(M: int, N: int, bm: int, bn: int):
    """Number of tile rows and tile columns: ceil(M/bm), ceil(N/bn)."""
    if bm < 1 or bn < 1 or M < 0 or N < 0:
        raise ValueError("block sizes must be >= 1 and shapes >= 0")
    return -(-M // bm), -(-N // bn)


def tile_scale(amax: float, eps: float = EPS):
    """Scale and reciprocal for one tile, from its largest magnitude.

    Returns ``(s, r)`` as Python floats holding float32 values:
    ``a = max(amax, fl32(eps))``, ``s = fl32(a / 448)``, ``r = fl32(1 / s)``.
    """
    if not math.isfinite(amax):
        raise ValueError("non-finite input is outside the quantizer's contract")
    a = max(amax, fl32(eps))
    s = fl32(a / E4M3_MAX)
    r = fl32(1.0 / s)
    return s, r


def quantize_tile(values, eps: float = EPS):
    """Quantize one tile given as a flat list of float32-representable floats.

    Returns ``(codes, s)``: the list of e4m3fn codes in the input order and
    the tile's float32 descale.
    """
    amax = max((abs(v) for v in values), default=0.0)
    s, r = tile_scale(amax, eps)
    codes = []
    for v in values:
        y = fl32(v * r)
        y = min(max(y, -E4M3_MAX), E4M3_MAX)
        codes.append(encode(y))
    return codes, s


def quantize_scalar(x_bits, M: int, N: int, bm: int, bn: int, eps: float = EPS):
    """Pure-Python scalar pipeline for tiny inputs.

    ``x_bits`` is a flat row-major sequence of M*N BF16 bit patterns.
    Returns ``(q, scale_inv)`` as flat row-major lists of codes and floats.
    """
    TM, TN = tile_grid(M, N, bm, bn)
    q = [0] * (M * N)
    scale_inv = [0.0] * (TM * TN)
    for ti in range(TM):
        for tj in range(TN):
            idx = [r * N + c
                   for r in range(ti * bm, min(M, (ti + 1) * bm))
                   for c in range(tj * bn, min(N, (tj + 1) * bn))]
            codes, s = quantize_tile([bf16_bits_to_float(x_bits[k]) for k in idx], eps)
            for k, c in zip(idx, codes):
                q[k] = c
            scale_inv[ti * TN + tj] = s
    return q, scale_inv


def tile_row_amax(x_abs: np.ndarray, TN: int, bn: int) -> np.ndarray:
    """Largest magnitude of each tile in one tile row (step: tile absmax).

    ``x_abs`` holds |x| of the tile row's valid elements, shape [rows, N].
    Columns past N are padded with zeros: |0| is never above a tile's
    maximum, so the padding leaves every maximum unchanged.
    """
    rows, N = x_abs.shape
    padded = np.zeros((rows, TN * bn), dtype=np.float64)
    padded[:, :N] = x_abs
    return padded.reshape(rows, TN, bn).max(axis=(0, 2))


def tile_scales_np(amax: np.ndarray, eps: float = EPS):
    """Vectorised ``tile_scale``: per-tile (s, r) as float64 arrays of float32 values."""
    a = np.maximum(amax, fl32(eps))
    s = (a / E4M3_MAX).astype(np.float32).astype(np.float64)      # fl32(a / 448)
    r = (1.0 / s).astype(np.float32).astype(np.float64)           # fl32(1 / s)
    return s, r


def scale_clamp_encode(x: np.ndarray, r_col: np.ndarray) -> np.ndarray:
    """Quantize values given each one's tile reciprocal: fl32(x*r), clamp, encode."""
    y = (x * r_col).astype(np.float32).astype(np.float64)          # fl32(x * r)
    y = np.minimum(np.maximum(y, -E4M3_MAX), E4M3_MAX)
    return encode_np(y)


def quantize(x_bits: np.ndarray, bm: int, bn: int, eps: float = EPS):
    """numpy pipeline: BF16 bits [M, N] -> (q uint8 [M, N], scale_inv float32 [TM, TN]).

    Works one tile row at a time; within a tile row all tiles go through the
    same array expressions (``tile_row_amax``, ``tile_scales_np``,
    ``scale_clamp_encode``), each element using its own tile's reciprocal.
    """
    x_bits = np.asarray(x_bits)
    if x_bits.ndim != 2 or x_bits.dtype != np.uint16:
        raise TypeError("x_bits must be a 2-D uint16 array of BF16 patterns")
    M, N = x_bits.shape
    TM, TN = tile_grid(M, N, bm, bn)
    q = np.empty((M, N), dtype=np.uint8)
    scale_inv = np.empty((TM, TN), dtype=np.float32)
    if M == 0 or N == 0:
        return q, scale_inv
    for ti in range(TM):
        r0, r1 = ti * bm, min(M, (ti + 1) * bm)
        x = bf16_bits_to_f64(x_bits[r0:r1])                       # exact widening
        if not np.all(np.isfinite(x)):
            raise ValueError("non-finite input is outside the quantizer's contract")
        amax = tile_row_amax(np.abs(x), TN, bn)                   # [TN]
        s, r = tile_scales_np(amax, eps)
        r_col = np.repeat(r, bn)[:N]                              # each column's tile
        q[r0:r1] = scale_clamp_encode(x, r_col)
        scale_inv[ti] = s.astype(np.float32)
    return q, scale_inv


def round_to_bf16(y: np.ndarray) -> np.ndarray:
    """Round float64 values (float32-representable, normal range) to the
    nearest BF16 value, ties to even: 8 significant bits."""
    y = np.asarray(y, dtype=np.float64)
    nz = y != 0
    a = np.abs(y[nz])
    if np.any(a < 2.0 ** -126) or np.any(a >= 2.0 ** 128):
        raise ValueError("BF16 rounding here covers the normal range only")
    frac, exp = np.frexp(y[nz])                    # y = frac * 2**exp, 0.5 <= |frac| < 1
    out = y.copy()
    out[nz] = np.ldexp(np.rint(frac * 256.0) / 256.0, exp)   # np.rint: half to even
    return out


def dequantize(q: np.ndarray, scale_inv: np.ndarray, bm: int, bn: int, out: str = "f32"):
    """Dequantization, the consumer side of the descale: x_hat = decode(q) * s.

    The page "fp8_kernel.py — FP8 量化内核" (section 1) calls the second
    output the descale, and the "vllm_fp8_utils.py" page (section 3) names
    it ``<weight>_scale_inv``: the stored value multiplies the FP8 value back.
    The product is rounded once to float32; ``out="bf16"`` rounds that
    float32 to the nearest BF16 (ties to even).  Returns float64 holding the
    float32 or BF16 values.
    """
    q = np.asarray(q, dtype=np.uint8)
    M, N = q.shape
    TM, TN = tile_grid(M, N, bm, bn)
    s = np.asarray(scale_inv, dtype=np.float32).astype(np.float64)
    if s.shape != (TM, TN):
        raise ValueError(f"scale_inv shape {s.shape} != {(TM, TN)}")
    s_full = np.repeat(np.repeat(s, bm, axis=0)[:M], bn, axis=1)[:, :N]
    y = (decode_np(q) * s_full).astype(np.float32).astype(np.float64)     # fl32(v * s)
    if out == "f32":
        return y
    if out == "bf16":
        return round_to_bf16(y)
    raise ValueError("out must be 'f32' or 'bf16'")


def local_grid(M: int, N: int, bm: int, bn: int, row_phase: int = 0, col_phase: int = 0):
    """Tile grid of an [M, N] sub-matrix whose element (0, 0) sits at
    (row_phase, col_phase) inside a tile of the full matrix's grid."""
    if not (0 <= row_phase < bm and 0 <= col_phase < bn):
        raise ValueError("phases must satisfy 0 <= phase < block")
    return -(-(row_phase + M) // bm), -(-(col_phase + N) // bn)


def tile_amax(x_bits: np.ndarray, bm: int, bn: int, row_phase: int = 0, col_phase: int = 0):
    """Largest |x| of each tile's part inside a sub-matrix (float64 [TMl, TNl]).

    For a sub-matrix cut out of a larger matrix (a shard), the maximum of
    each tile of the full matrix is the max over the shards of these partial
    maxima; the tile maximum is the first step of the blockwise cast (page
    "fp8_kernel.py — FP8 量化内核", section 2).
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, N = x_bits.shape
    TM, TN = local_grid(M, N, bm, bn, row_phase, col_phase)
    out = np.zeros((TM, TN), dtype=np.float64)
    if M == 0 or N == 0:
        return out
    a = np.abs(bf16_bits_to_f64(x_bits))
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite input is outside the quantizer's contract")
    # local tile (ti, tj) covers rows [ti*bm - row_phase, (ti+1)*bm - row_phase)
    # and columns [tj*bn - col_phase, (tj+1)*bn - col_phase) of the sub-matrix,
    # clipped to it; every local tile holds at least one element
    for ti in range(TM):
        r0, r1 = max(0, ti * bm - row_phase), min(M, (ti + 1) * bm - row_phase)
        for tj in range(TN):
            c0, c1 = max(0, tj * bn - col_phase), min(N, (tj + 1) * bn - col_phase)
            out[ti, tj] = a[r0:r1, c0:c1].max()
    return out


def quantize_with_amax(x_bits: np.ndarray, bm: int, bn: int, amax: np.ndarray,
                       row_phase: int = 0, col_phase: int = 0, eps: float = EPS):
    """Quantize a sub-matrix with given whole-tile maxima (float64 [TMl, TNl]):
    scales and reciprocals from ``amax`` exactly as in ``tile_scales_np``,
    then each element scaled by its tile's reciprocal, clamped and encoded.
    Returns (q uint8 [M, N], scale_inv float32 [TMl, TNl])."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, N = x_bits.shape
    TM, TN = local_grid(M, N, bm, bn, row_phase, col_phase)
    amax = np.asarray(amax, dtype=np.float64)
    if amax.shape != (TM, TN):
        raise ValueError(f"amax shape {amax.shape} != {(TM, TN)}")
    s, r = tile_scales_np(amax, eps)
    q = np.empty((M, N), dtype=np.uint8)
    if M and N:
        rows = (np.arange(M) + row_phase) // bm
        cols = (np.arange(N) + col_phase) // bn
        r_full = r[rows][:, cols]
        q[:] = scale_clamp_encode(bf16_bits_to_f64(x_bits), r_full)
    return q, s.astype(np.float32)
