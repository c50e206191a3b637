"""OCP FP8 E4M3 ("float8_e4m3fn") from the format's definition (test infrastructure only).

The page "fp8_kernel.py — FP8 量化内核" (background section) names the target
type ``float8_e4m3fn``.  Its definition (the OCP 8-bit floating point format):

* 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
* exponent field 0 holds subnormals ``m/8 * 2**-6``;
* no infinities; the exponent field 1111 with mantissa 111 is NaN
  (codes 0x7F and 0xFF), so the largest finite magnitude is
  ``1.75 * 2**8 = 448`` (code 0x7E);
* conversion rounds to nearest, ties to even (even = mantissa LSB 0).

The encoders accept finite values with ``|v| <= 448`` only; the quantizer
clamps to that range before it encodes, so nothing else ever reaches them.
"""

import math

import numpy as np

BIAS = 7
MAX_FINITE = 448.0
MIN_NORMAL = 2.0 ** -6          # code 0x08
SUBNORMAL_STEP = 2.0 ** -9      # code 0x01
NAN_CODES = (0x7F, 0xFF)


def decode(code: int) -> float:
    """Value of an 8-bit code."""
    code &= 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * SUBNORMAL_STEP
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - BIAS)


def decode_np(codes) -> np.ndarray:
    """Vectorised ``decode`` (float64 out)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2((e - BIAS).astype(np.float64))
    sub = m * SUBNORMAL_STEP
    val = sign * np.where(e == 0, sub, normal)
    return np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, val)


def encode(v: float) -> int:
    """Round one finite value with ``|v| <= 448`` to its e4m3fn code (RNE).

    The sign bit is copied from ``v``, so -0.0 and negatives that round to
    zero give 0x80.
    """
    if not math.isfinite(v) or abs(v) > MAX_FINITE:
        raise ValueError(f"e4m3fn encoder takes finite |v| <= 448, got {v!r}")
    sign = 0x80 if math.copysign(1.0, v) < 0 else 0x00
    a = abs(v)
    if a < MIN_NORMAL:
        # Subnormal range: the grid is uniform with step 2**-9, so the code is
        # the nearest integer multiple of the step.  a*512 is exact and
        # Python's round() on a float rounds half to even.  A result of 8
        # lands on 0x08, the smallest normal, which is the right code.
        return sign | int(round(a * 512.0))
    frac2, exp2 = math.frexp(a)              # a = frac2 * 2**exp2, frac2 in [0.5, 1)
    exponent = exp2 - 1                      # a = sig * 2**exponent, sig in [1, 2)
    sig = 2.0 * frac2
    mant = int(round((sig - 1.0) * 8.0))     # exact product; ties to even
    if mant == 8:                            # rounded up into the next binade
        exponent += 1
        mant = 0
    return sign | ((exponent + BIAS) << 3) | mant


def encode_np(y) -> np.ndarray:
    """Vectorised ``encode`` over float64 values (each finite, |y| <= 448)."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)) or np.any(np.abs(y) > MAX_FINITE):
        raise ValueError("e4m3fn encoder takes finite |v| <= 448")
    sign = np.where(np.signbit(y), 0x80, 0x00).astype(np.int64)
    a = np.abs(y)
    # subnormal branch
    sub_code = np.rint(a * 512.0).astype(np.int64)       # np.rint: half to even
    # normal branch
    frac2, exp2 = np.frexp(np.where(a < MIN_NORMAL, 1.0, a))
    exponent = exp2.astype(np.int64) - 1
    mant = np.rint((2.0 * frac2 - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8
    exponent = exponent + carry
    mant = np.where(carry, 0, mant)
    norm_code = ((exponent + BIAS) << 3) | mant
    mag = np.where(a < MIN_NORMAL, sub_code, norm_code)
    return (sign | mag).astype(np.uint8)
