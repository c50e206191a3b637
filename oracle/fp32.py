"""float32 rounding and BF16 widening for the oracle (test infrastructure only).

The quantizer's arithmetic is float32 (the Triton kernel on the page
"fp8_kernel.py — FP8 量化内核", section 2, computes the scale and the scaled
values on the loaded block; the reading taken here is float32 with correctly
rounded division).  The oracle keeps values in float64 and rounds to float32
explicitly after each operation.
"""

import struct

import numpy as np


def fl32(v: float) -> float:
    """Round a Python float (binary64) to the nearest binary32, ties to even.

    ``struct`` performs the C conversion ``(float)v``, which rounds to nearest
    even under the default rounding mode and keeps the sign of zero.
    """
    return struct.unpack("<f", struct.pack("<f", v))[0]


def fl32_np(v: np.ndarray) -> np.ndarray:
    """Vectorised ``fl32``: float64 in, float64 out holding float32 values."""
    return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def f32_bits(v: float) -> int:
    """The 32-bit pattern of a float32 value (given as a Python float)."""
    return struct.unpack("<I", struct.pack("<f", v))[0]


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen BF16 bit patterns (uint16) to float64, exactly.

    A BF16 value is the upper half of the float32 with the same bits, so the
    widening shifts the pattern into the high 16 bits of a float32 word.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def bf16_bits_to_float(bits: int) -> float:
    """Scalar BF16 widening (pure Python)."""
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
